// Batch-1 decode path of the MoE layer (gfx950): matrix-vector kernels that
// stream the packed 4-bit weights of the k routed experts and the shared
// expert at HBM rate, with wave reductions and no matrix cores.  The Lily
// pages run batch-1 decode on the vector ALUs because one token gives no
// weight reuse, so the pass is bound by memory bandwidth (page "Perplexity's
// Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple Silicon", section "Why
// prefill and decode get different treatment").
//
// Two kernels per layer:
//   decode_gateup_kernel  top-k of the token's logits (wave 0 of every block,
//                         DPP maxima; block 0 also writes the routing
//                         outputs), then h_j[n] = silu(W_gate,j[n] . x) *
//                         (W_up,j[n] . x) for the shared expert and the k
//                         routed ones, fp32.  The shared expert's rows come
//                         first in the work order and their loads are issued
//                         before the routing result is waited for;
//   decode_down_kernel    y[i] = sum_j w_j (W_down,j[i] . h_j) + W_sdown[i] . h_s,
//                         one block per 4 output rows, one wave per 64
//                         chunks of the concatenated hidden vector.
//
// The 4-bit decode uses the factored form of one affine group,
//   sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i,
// so the codes are converted to fp32 and multiplied by x, and the scale and
// bias are applied once per 32-element chunk.  No bf16 rounding of weights.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kDecThreads = 256;  // 4 waves per block
constexpr int kDecPairs = 2;      // (gate, up) row pairs per wave
constexpr int kDownRows = 4;      // output rows per down block

struct DecodeArgs {
    const float *logits;  // [1][E] or null (routing given in r)
    const uint16_t *x;    // [1][d]
    moe_weights w;
    moe_routing r;
    int d, E, k, F, Fs, G, Fmax;
    float *h;             // [k+1][Fmax] fp32 workspace: slots 0..k-1 routed, k shared
    uint16_t *y;          // [1][d]
};

// routing outputs of the single token (block 0 only): ids, weights, the
// one-row-per-expert histogram, its scan, the sorted order and the tiles
__device__ void decode_write_routing(const DecodeArgs &a, const int *s_ids, const float *s_w)
{
    const int tid = threadIdx.x;
    const moe_routing &r = a.r;
    for (int j = tid; j < a.k; j += blockDim.x) {
        r.topk_ids[j] = s_ids[j];
        r.topk_w[j] = s_w[j];
        int rank = 0;  // sorted position = number of chosen experts with a lower id
        for (int i = 0; i < a.k; ++i) rank += s_ids[i] < s_ids[j];
        r.perm[rank] = j;
        r.inv_perm[j] = rank;
        r.tile_expert[rank] = s_ids[j];
        r.tile_row0[rank] = rank;
        r.tile_rows[rank] = 1;
    }
    for (int e = tid; e <= a.E; e += blockDim.x) {
        int below = 0, hit = 0;
        for (int i = 0; i < a.k; ++i) { below += s_ids[i] < e; hit += s_ids[i] == e; }
        if (e < a.E) r.counts[e] = hit;
        r.offsets[e] = below;
    }
    if (tid == 0) *r.num_tiles = a.k;
}

// raw operands of one (gate, up) row pair for one 32-element chunk
struct PairRaw {
    uint4 qg, qu;
    uint16_t sg, bg, su, bu;
};

__device__ __forceinline__ void load_pair(PairRaw &r, const moe_qmat &mg, const moe_qmat &mu, size_t row,
                                          int c, int d, int G)
{
    const size_t qo = row * (size_t)(d >> 1) + (size_t)c * 16;
    r.qg = *reinterpret_cast<const uint4 *>(mg.q + qo);
    r.qu = *reinterpret_cast<const uint4 *>(mu.q + qo);
    const size_t gi = row * (size_t)(d / G) + (size_t)(c * 32) / G;
    r.sg = mg.s[gi]; r.bg = mg.b[gi];
    r.su = mu.s[gi]; r.bu = mu.b[gi];
}

// NCH = 32-element chunks of x per lane (d <= 2048 * NCH)
template <int NCH>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs a)
{
    __shared__ int s_ids[kMaxE];
    __shared__ float s_w[kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nchunk = a.d >> 5;
    const int npairs = a.Fs + a.k * a.F;
    const int p0 = (blockIdx.x * (kDecThreads / kWave) + wave) * kDecPairs;

    // x chunks of this lane: chunk c = lane + 64 i covers x[32c, 32c+32)
    uint4 xr[NCH][4];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(a.x + (size_t)c * 32);
#pragma unroll
            for (int v = 0; v < 4; ++v) xr[i][v] = xp[v];
        }
    }
    // shared-expert rows do not depend on the routing: load them first
    PairRaw raw[kDecPairs][NCH];
#pragma unroll
    for (int pi = 0; pi < kDecPairs; ++pi) {
        const int p = p0 + pi;
        if (p < a.Fs) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = lane + 64 * i;
                if (c < nchunk) load_pair(raw[pi][i], a.w.sgate, a.w.sup, (size_t)p, c, a.d, a.G);
            }
        }
    }
    if (a.logits) {
        if (wave == 0) {
            TopK tk;
            wave_topk(load_logits(a.logits, a.E), a.E, a.k, tk);
            float ex[4], part = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = lane + 64 * c;
                ex[c] = (j < a.k) ? expf(tk.logit[c] - tk.lmax) : 0.f;
                part += ex[c];
            }
            const float inv = 1.0f / wave_sum(part);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = lane + 64 * c;
                if (j < a.k) { s_ids[j] = tk.id[c]; s_w[j] = ex[c] * inv; }
            }
        }
        __syncthreads();
        if (blockIdx.x == 0) decode_write_routing(a, s_ids, s_w);
    } else {
        for (int j = tid; j < a.k; j += kDecThreads) s_ids[j] = a.r.topk_ids[j];
        __syncthreads();
    }
#pragma unroll
    for (int pi = 0; pi < kDecPairs; ++pi) {
        const int p = p0 + pi;
        if (p >= a.Fs && p < npairs) {
            const int j = (p - a.Fs) / a.F, n = (p - a.Fs) - j * a.F;
            const size_t row = (size_t)s_ids[j] * a.F + n;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = lane + 64 * i;
                if (c < nchunk) load_pair(raw[pi][i], a.w.gate, a.w.up, row, c, a.d, a.G);
            }
        }
    }
    float accg[kDecPairs], accu[kDecPairs];
#pragma unroll
    for (int pi = 0; pi < kDecPairs; ++pi) { accg[pi] = 0.f; accu[pi] = 0.f; }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c >= nchunk) continue;
        float xv[32], xs = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint32_t wd[4] = {xr[i][v].x, xr[i][v].y, xr[i][v].z, xr[i][v].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[8 * v + 2 * q] = bf16_to_f32(wd[q] & 0xFFFFu);
                xv[8 * v + 2 * q + 1] = bf16_to_f32(wd[q] >> 16);
            }
        }
#pragma unroll
        for (int q = 0; q < 32; ++q) xs += xv[q];
#pragma unroll
        for (int pi = 0; pi < kDecPairs; ++pi) {
            const PairRaw &r = raw[pi][i];
            float dg = 0.f, du = 0.f;
            dg = dot8_codes(r.qg.x, xv + 0, dg);
            dg = dot8_codes(r.qg.y, xv + 8, dg);
            dg = dot8_codes(r.qg.z, xv + 16, dg);
            dg = dot8_codes(r.qg.w, xv + 24, dg);
            du = dot8_codes(r.qu.x, xv + 0, du);
            du = dot8_codes(r.qu.y, xv + 8, du);
            du = dot8_codes(r.qu.z, xv + 16, du);
            du = dot8_codes(r.qu.w, xv + 24, du);
            accg[pi] += bf16_to_f32(r.sg) * dg + bf16_to_f32(r.bg) * xs;
            accu[pi] += bf16_to_f32(r.su) * du + bf16_to_f32(r.bu) * xs;
        }
    }
#pragma unroll
    for (int pi = 0; pi < kDecPairs; ++pi) {
        const int p = p0 + pi;
        const float g = wave_sum(accg[pi]);
        const float u = wave_sum(accu[pi]);
        if (lane == 0 && p < npairs) {
            int j, n;
            if (p < a.Fs) { j = a.k; n = p; }
            else { j = (p - a.Fs) / a.F; n = (p - a.Fs) - j * a.F; }
            a.h[(size_t)j * a.Fmax + n] = silu(g) * u;
        }
    }
}

// One block = kDownRows output rows; wave w takes the 32-wide chunks
// w*64 + lane, w*64 + lane + 64*nw, ... of [h_0 .. h_{k-1}, h_s].
__global__ void decode_down_kernel(DecodeArgs a)
{
    __shared__ float red[16][kDownRows];
    __shared__ int s_ids[kMaxE];
    __shared__ float s_w[kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nw = blockDim.x >> 6;
    for (int j = tid; j < a.k; j += blockDim.x) { s_ids[j] = a.r.topk_ids[j]; s_w[j] = a.r.topk_w[j]; }
    __syncthreads();
    const int row0 = blockIdx.x * kDownRows;
    const int cF = a.F >> 5, cFs = a.Fs >> 5;
    const int nchunks = a.k * cF + cFs;
    float acc[kDownRows];
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) acc[r] = 0.f;
    for (int c = wave * kWave + lane; c < nchunks; c += nw * kWave) {
        int j, f0, Fw;
        const moe_qmat *m;
        size_t ebase;
        float wj;
        if (c < a.k * cF) {
            j = c / cF; f0 = (c - j * cF) * 32; Fw = a.F; m = &a.w.down;
            ebase = (size_t)s_ids[j] * a.d;
            wj = s_w[j];
        } else {
            j = a.k; f0 = (c - a.k * cF) * 32; Fw = a.Fs; m = &a.w.sdown;
            ebase = 0;
            wj = 1.0f;
        }
        uint4 q[kDownRows];
        uint16_t sb[kDownRows][2];
        const int grp = f0 / a.G;
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) {
            const size_t row = ebase + min(row0 + r, a.d - 1);
            q[r] = *reinterpret_cast<const uint4 *>(m->q + row * (size_t)(Fw >> 1) + (f0 >> 1));
            const size_t gi = row * (size_t)(Fw / a.G) + grp;
            sb[r][0] = m->s[gi];
            sb[r][1] = m->b[gi];
        }
        float hv[32], hs = 0.f;
        const float4 *hp = reinterpret_cast<const float4 *>(a.h + (size_t)j * a.Fmax + f0);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float4 t = hp[v];
            hv[4 * v] = t.x; hv[4 * v + 1] = t.y; hv[4 * v + 2] = t.z; hv[4 * v + 3] = t.w;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) hs += hv[i];
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) {
            float dq = 0.f;
            dq = dot8_codes(q[r].x, hv + 0, dq);
            dq = dot8_codes(q[r].y, hv + 8, dq);
            dq = dot8_codes(q[r].z, hv + 16, dq);
            dq = dot8_codes(q[r].w, hv + 24, dq);
            acc[r] += wj * (bf16_to_f32(sb[r][0]) * dq + bf16_to_f32(sb[r][1]) * hs);
        }
    }
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == 0) red[wave][r] = v;
    }
    __syncthreads();
    if (tid < kDownRows && row0 + tid < a.d) {
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[w][tid];
        a.y[row0 + tid] = f32_to_bf16(v);
    }
}

hipError_t launch_decode(const Plan &p, const float *logits, const uint16_t *x,
                         const moe_weights &w, const moe_routing &r, uint16_t *y, void *ws,
                         hipStream_t s, EventTrace *tr)
{
    DecodeArgs a;
    a.logits = logits;
    a.x = x;
    a.w = w;
    a.r = r;
    a.d = p.d; a.E = p.E; a.k = p.k; a.F = p.F; a.Fs = p.Fs; a.G = p.G;
    a.Fmax = p.F > p.Fs ? p.F : p.Fs;
    a.h = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_dech);
    a.y = y;
    const int npairs = p.k * p.F + p.Fs;
    const int per_block = (kDecThreads / kWave) * kDecPairs;
    const int nb1 = (npairs + per_block - 1) / per_block;
    const int nch = (p.d / 32 + kWave - 1) / kWave;
    if (nch <= 1)
        launch(tr, decode_gateup_kernel<1>, dim3(nb1), dim3(kDecThreads), 0, s, a);
    else if (nch <= 2)
        launch(tr, decode_gateup_kernel<2>, dim3(nb1), dim3(kDecThreads), 0, s, a);
    else if (nch <= 4)
        launch(tr, decode_gateup_kernel<4>, dim3(nb1), dim3(kDecThreads), 0, s, a);
    else
        launch(tr, decode_gateup_kernel<8>, dim3(nb1), dim3(kDecThreads), 0, s, a);
    const int nchunks = p.k * (p.F >> 5) + (p.Fs >> 5);
    int nw = (nchunks + kWave - 1) / kWave;
    nw = nw < 1 ? 1 : (nw > 16 ? 16 : nw);
    const int nb2 = (p.d + kDownRows - 1) / kDownRows;
    launch(tr, decode_down_kernel, dim3(nb2), dim3(nw * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
