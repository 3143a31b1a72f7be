// Device-side helpers shared by the gfx950 kernels of the MoE layer:
// bf16 conversion, the 4-bit affine decode, wave-wide reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// two fp32 -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32);
// `lo` lands in bits 0..15
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// Decode 8 consecutive 4-bit codes (one dword; element 2m in the low nibble
// of byte m) of one affine group to 4 packed bf16 pairs, element 2r in the
// low half of out[r].  Value = bf16_rne(fma(s, q, b)); s*q is exact in fp32,
// so the fma rounds the exact s*q + b once.
// Unpacking: a byte holding one code q (0..15) read as an OCP fp8 e4m3
// value is q * 2^-9 exactly (codes 0..7 are the denormals m * 2^-9, codes
// 8..15 the first normal binade (8 + m) * 2^-9), so one v_cvt_pk_f32_fp8
// turns two isolated codes into fp32, and fma(512 s, q 2^-9, b) equals
// fma(s, q, b) bit for bit (scaling by powers of two is exact for any scale
// below 2^119).
constexpr float kFp8CodeScale = 512.0f;

__device__ __forceinline__ void dequant8_bf16(uint32_t v, float s, float b, uint32_t out[4])
{
    const float s9 = s * kFp8CodeScale;
    const uint32_t lo = v & 0x0F0F0F0Fu;         // elements 0,2,4,6
    const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;  // elements 1,3,5,7
    const auto l01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // elements 0, 2
    const auto l23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // elements 4, 6
    const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);  // elements 1, 3
    const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);   // elements 5, 7
    out[0] = pack_bf16x2(__builtin_fmaf(s9, l01[0], b), __builtin_fmaf(s9, h01[0], b));
    out[1] = pack_bf16x2(__builtin_fmaf(s9, l01[1], b), __builtin_fmaf(s9, h01[1], b));
    out[2] = pack_bf16x2(__builtin_fmaf(s9, l23[0], b), __builtin_fmaf(s9, h23[0], b));
    out[3] = pack_bf16x2(__builtin_fmaf(s9, l23[1], b), __builtin_fmaf(s9, h23[1], b));
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Give each XCD an equal contiguous range of the `total` logical
// blocks, so that consecutive logical blocks (the column blocks of one GEMM
// tile, then the next tile of the same expert; neighbouring output rows of
// a matrix-vector product) run on the same XCD and share its L2.  The grid
// must hold at least 8 ceil(total / 8) blocks (a multiple of 8 >= total);
// -1: a padding block with no work.
__device__ __forceinline__ int xcd_logical_block(int bid, int total)
{
    const int per = (total + 7) >> 3;
    const int i = bid >> 3;
    if (i >= per) return -1;
    const int L = (bid & 7) * per + i;
    return L < total ? L : -1;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// sum over the 64 lanes, broadcast to all: butterflies inside rows of 16
// (quad permutes, row rotates), then row broadcasts 15 and 31 into lane 63
// a.lo * b.lo + a.hi * b.hi + c for bf16 pairs a, b (fp32 products and sum)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<0xB1>(v);         // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);         // quad_perm [2,3,0,1]
    v += dpp_f32<0x124>(v);        // row_ror:4
    v += dpp_f32<0x128>(v);        // row_ror:8  -> every lane holds its row sum
    v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Total order on finite fp32 logits as unsigned keys: larger logit -> larger
// key; -0 is folded into +0 first so that the two compare equal.
__device__ __forceinline__ uint32_t logit_key(float l)
{
    uint32_t u = (l == 0.0f) ? 0u : __float_as_uint(l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// DPP move of v within rows of 16 lanes / across rows; lanes with no source
// get 0, the identity of an unsigned max.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// max over the 64 lanes, broadcast to all (DPP row shifts, then row
// broadcasts 15 and 31 carry the row maxima to lane 63)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0x111>(v));        // row_shr:1
    v = max(v, dpp_u32<0x112>(v));        // row_shr:2
    v = max(v, dpp_u32<0x114>(v));        // row_shr:4
    v = max(v, dpp_u32<0x118>(v));        // row_shr:8
    v = max(v, dpp_u32<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
    v = max(v, dpp_u32<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one row of E <= 256 logits by one wave (rounds of the selection
// below).  Selected (id, logit) of round j end up in lane j % 64, register
// j / 64.
struct TopK {
    int id[4];
    float logit[4];
    float lmax;
};

// logits of experts 4 lane .. 4 lane + 3 of one row (rows past E read as 0)
struct LogitQuad {
    float v[4];
};

__device__ __forceinline__ LogitQuad load_logits(const float *__restrict__ L, int E)
{
    const int lane = threadIdx.x & 63;
    LogitQuad q;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = 4 * lane + c;
        q.v[c] = e < E ? L[e] : 0.f;
    }
    return q;
}

// The wave's keys for the selection rounds: lane l holds experts 4l .. 4l+3,
// sorted once per lane by key descending, ties to the lower expert (key 0 =
// no expert), so the lane's current largest key is k[0] and its expert slot
// s[0].  A round is then one wave max of the lane heads, the lowest lane
// holding it (ballot, find-first: lane order is expert order, so ties go to
// the lower id), and a shift of that lane's list.
struct LaneKeys {
    uint32_t k[4];
    int s[4];
};

__device__ __forceinline__ void lane_keys_cmpx(LaneKeys &t, int a, int b)
{
    const bool sw = t.k[a] < t.k[b] || (t.k[a] == t.k[b] && t.s[a] > t.s[b]);
    const uint32_t ka = t.k[a], kb = t.k[b];
    const int sa = t.s[a], sb = t.s[b];
    t.k[a] = sw ? kb : ka; t.k[b] = sw ? ka : kb;
    t.s[a] = sw ? sb : sa; t.s[b] = sw ? sa : sb;
}

__device__ __forceinline__ LaneKeys lane_keys(const uint32_t (&key)[4])
{
    LaneKeys t;
#pragma unroll
    for (int c = 0; c < 4; ++c) { t.k[c] = key[c]; t.s[c] = c; }
    // 4-input sorting network
    lane_keys_cmpx(t, 0, 1); lane_keys_cmpx(t, 2, 3);
    lane_keys_cmpx(t, 0, 2); lane_keys_cmpx(t, 1, 3);
    lane_keys_cmpx(t, 1, 2);
    return t;
}

// One selection round: the largest remaining key m and the lane holding it
// (lowest lane on ties); that lane drops its head.  The expert is
// 4 * lane + (its s[0] before the drop), read only when needed.
__device__ __forceinline__ int topk_round(LaneKeys &t, uint32_t &m, int &slot)
{
    const int lane = threadIdx.x & 63;
    m = wave_max_u32(t.k[0]);
    const uint64_t holders = __ballot(t.k[0] == m);
    const int wl = __ffsll((unsigned long long)holders) - 1;
    slot = t.s[0];
    if (lane == wl) {
        t.k[0] = t.k[1]; t.k[1] = t.k[2]; t.k[2] = t.k[3]; t.k[3] = 0u;
        t.s[0] = t.s[1]; t.s[1] = t.s[2]; t.s[2] = t.s[3];
    }
    return wl;
}

__device__ __forceinline__ void wave_topk(const LogitQuad &lq, int E, int k, TopK &out)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = 4 * lane + c;
        key[c] = (e < E) ? logit_key(lq.v[c]) : 0u;  // 0: no expert (finite keys are > 0)
    }
    LaneKeys t = lane_keys(key);
#pragma unroll
    for (int c = 0; c < 4; ++c) { out.id[c] = 0; out.logit[c] = 0.f; }
    out.lmax = 0.f;
    for (int j = 0; j < k; ++j) {
        uint32_t m;
        int slot;
        const int wl = topk_round(t, m, slot);
        const int id = 4 * wl + __builtin_amdgcn_readlane(slot, wl);
        const float l = key_logit(m);
        if (j == 0) out.lmax = l;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (j == lane + 64 * c) { out.id[c] = id; out.logit[c] = l; }
    }
}

// Expert of rank j (0-based, ties to the lower id) among the wave's keys:
// rounds 0 .. j of the selection above, nothing more.
__device__ __forceinline__ int wave_rank_expert(const uint32_t (&key)[4], int j)
{
    LaneKeys t = lane_keys(key);
    uint32_t m;
    int slot;
    for (int r = 0; r < j; ++r) topk_round(t, m, slot);
    const int wl = topk_round(t, m, slot);
    return 4 * wl + __builtin_amdgcn_readlane(slot, wl);
}

__device__ __forceinline__ float silu(float z)
{
    return z / (1.0f + __expf(-z));
}

}  // namespace moe
