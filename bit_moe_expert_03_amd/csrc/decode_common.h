// Pieces shared by the matrix-vector kernels of the decode path (gfx950):
// the packed 4-bit dot products in factored form and the raw row operands.
//
// The 4-bit dot products use the factored form of one affine group,
//   sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i,
// with the codes turned into exact bf16 values 128 + q (one byte permute
// against the constant byte 0x43 yields two of them) and multiplied with
// v_dot2_f32_bf16 (fp32 accumulation); the offset is folded into the bias
// term: s * sum (128 + q_i) x_i + (b - 128 s) * sum x_i.  The codes of one
// 32-bit word pair up as (e0, e2), (e4, e6), (e1, e3), (e5, e7); the vector
// operand is permuted once per lane into the same order.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---- packed 4-bit dot products ---------------------------------------------

constexpr uint32_t kBf16Ones = 0x3F803F80u;  // the bf16 pair (1.0, 1.0)

// 32 elements of a bf16 vector as the bf16 pairs in the order dot_codes32_rows()
// pairs the codes, and their fp32 sum
struct VecChunk {
    uint32_t p[16];
    float sum;
};

__device__ __forceinline__ void vec_chunk(const uint4 (&w)[4], VecChunk &v)
{
    v.sum = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = w[g].x, w1 = w[g].y, w2 = w[g].z, w3 = w[g].w;  // (x0,x1) .. (x6,x7)
        v.p[4 * g + 0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);  // (x0, x2)
        v.p[4 * g + 1] = __builtin_amdgcn_perm(w3, w2, 0x05040100u);  // (x4, x6)
        v.p[4 * g + 2] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);  // (x1, x3)
        v.p[4 * g + 3] = __builtin_amdgcn_perm(w3, w2, 0x07060302u);  // (x5, x7)
        // the chunk sum as dot products with the bf16 pair (1, 1), fp32 accumulation
        v.sum = dot2_bf16(w0, kBf16Ones, v.sum);
        v.sum = dot2_bf16(w1, kBf16Ones, v.sum);
        v.sum = dot2_bf16(w2, kBf16Ones, v.sum);
        v.sum = dot2_bf16(w3, kBf16Ones, v.sum);
    }
}

// sum over the chunk of (128 + q_i) * v_i for the 32 codes of each of NR
// rows against the same chunk (one dot2 chain per row; the decode kernels
// keep two or more waves per SIMD, which hides the chain's latency --
// measured: interleaving the rows' chains by hand gained nothing there)
template <int NR>
__device__ __forceinline__ void dot_codes32_rows(const uint4 (&q)[NR], const VecChunk &v, float (&out)[NR])
{
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const uint32_t wd[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t lo = wd[g] & 0x0F0F0F0Fu;         // e0, e2, e4, e6 (one per byte)
            const uint32_t hi = (wd[g] >> 4) & 0x0F0F0F0Fu;  // e1, e3, e5, e7
            // bytes (e, 0x43, e', 0x43): the bf16 pair (128 + e, 128 + e')
            acc = dot2_bf16(__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u), v.p[4 * g + 0], acc);
            acc = dot2_bf16(__builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u), v.p[4 * g + 1], acc);
            acc = dot2_bf16(__builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u), v.p[4 * g + 2], acc);
            acc = dot2_bf16(__builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u), v.p[4 * g + 3], acc);
        }
        out[r] = acc;
    }
}

// one chunk's share of an affine-group dot product: s * sum q v + b * sum v
__device__ __forceinline__ float chunk_term(float dq128, const VecChunk &v, uint16_t s, uint16_t b)
{
    const float sf = bf16_to_f32(s), bf = bf16_to_f32(b);
    return sf * dq128 + (bf - 128.0f * sf) * v.sum;
}

// raw operands of one row for one 32-element chunk
struct RowRaw {
    uint4 q;
    uint16_t s, b;
};

__device__ __forceinline__ void load_row(RowRaw &r, const moe_qmat &m, size_t row, int c, int d, int G)
{
    r.q = *reinterpret_cast<const uint4 *>(m.q + row * (size_t)(d >> 1) + (size_t)c * 16);
    const size_t gi = row * (size_t)(d / G) + (size_t)(c * 32) / G;
    r.s = m.s[gi];
    r.b = m.b[gi];
}

// ---- routing outputs -----------------------------------------------------------

// Routing outputs of the batch from the chosen ids and weights of its
// A = T k assignments (a = t k + j): per-expert counts, their exclusive scan
// (offsets) and the scan of the used-expert flags (tile index) by wave 0,
// then the stable sorted position of each assignment, offsets[e] plus the
// number of earlier assignments of the same expert.  An expert is chosen at
// most once per token, so it has at most T <= tile_m rows and one tile.
__device__ inline void decode_write_routing(const moe_routing &r, int T, int E, int k, const int *s_ids,
                                           const float *s_w)
{
    __shared__ int cnt[kMaxE], off[kMaxE + 1], tix[kMaxE + 1];
    const int tid = threadIdx.x;
    const int A = T * k;
    for (int e = tid; e < kMaxE; e += blockDim.x) {
        int hit = 0;
        if (e < E)
            for (int i = 0; i < A; ++i) hit += s_ids[i] == e;
        cnt[e] = hit;
    }
    __syncthreads();
    if (tid < kWave) {  // exclusive scans over the (at most 256) experts, 4 per lane
        int v[4], u[4], sv = 0, su = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = cnt[4 * tid + i];
            u[i] = v[i] > 0;
            sv += v[i];
            su += u[i];
        }
        int iv = sv, iu = su;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int x = __shfl_up(iv, o, kWave), y = __shfl_up(iu, o, kWave);
            if (tid >= o) { iv += x; iu += y; }
        }
        int rv = iv - sv, ru = iu - su;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            off[4 * tid + i] = rv;
            tix[4 * tid + i] = ru;
            rv += v[i];
            ru += u[i];
        }
        if (tid == kWave - 1) { off[kMaxE] = rv; tix[kMaxE] = ru; }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += blockDim.x) {
        const int o = e < E ? off[e] : A;
        r.offsets[e] = o;
        if (e < E) {
            r.counts[e] = cnt[e];
            if (cnt[e]) {
                r.tile_expert[tix[e]] = e;
                r.tile_row0[tix[e]] = o;
                r.tile_rows[tix[e]] = cnt[e];
            }
        } else {
            *r.num_tiles = tix[kMaxE];
        }
    }
    for (int i = tid; i < A; i += blockDim.x) {
        const int e = s_ids[i];
        int rank = off[e];
        for (int i2 = 0; i2 < i; ++i2) rank += s_ids[i2] == e;
        r.topk_ids[i] = e;
        r.topk_w[i] = s_w[i];
        r.perm[rank] = i;
        r.inv_perm[i] = rank;
    }
}

}  // namespace moe
