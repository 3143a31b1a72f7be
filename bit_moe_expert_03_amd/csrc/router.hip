// Router projection of the MoE layer (gfx950): logits = x W_r (+ bias) on the
// bf16 matrix cores, the step in front of the routing (page "Perplexity's
// Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple Silicon", section
// "What Lily actually does": each token's router picks its experts).
//
// W_r is fp32 [d][E].  It is split once per weight set into two bf16
// matrices, hi = bf16(W) and lo = bf16(W - hi) (W - hi is exact in fp32), so
// that x W = x hi + x lo up to |W - hi - lo| <= 2^-17 |W| per weight; x is
// bf16 already, every product of two bf16 values is exact in fp32 and the
// matrix cores accumulate in fp32.  Packed layout: [2][Epad][d] bf16 (hi
// rows, then lo rows), expert-major so that each lane's MFMA operand is 16
// contiguous bytes; Epad = E rounded up to 64, padding rows zero.
//
// router_gemm_kernel: one block = 128 tokens x EX experts (64, or 32 for
// batches that would not fill the chip) over a K range, eight waves: wave w
// takes the 32 tokens of tile w % 4 against the block's experts (EX / 32
// tiles of 32) over half of every 64-wide K chunk (its 16-wide sub-steps
// 2 (w / 4) and 2 (w / 4) + 1), so that two waves share each SIMD and hide
// each other's barrier and LDS latency; the two halves' sums are added at
// the end (half 0 + half 1).  Per K chunk the block's router rows (hi and
// lo, EX experts) and its 128 activation rows (16 KB) are copied global ->
// LDS (global_load_lds_dwordx4) into a ring of four stages, four chunks
// ahead of the MFMAs that use them; each router row is read from L2 once per
// 128 tokens.  v_mfma_f32_32x32x16_bf16 with the
// router as the first operand, so lane l holds token l % 32 of the wave's
// tile and register r of an expert tile holds expert 8 (r / 4) + 4 (l / 32)
// + r % 4 of it.  When the grid would be small, K is split into KS ranges
// whose partial logits a second kernel sums in range order (deterministic),
// adding the bias; with KS = 1 the GEMM writes the logits itself.
#include <type_traits>

#include "gemm_common.h"

namespace moe {

constexpr int kRouterThreads = 512;  // 8 waves per block: 4 token tiles x 2 halves of each K chunk

__global__ __launch_bounds__(256) void router_pack_kernel(const float *__restrict__ W, int d, int E, int Epad,
                                                          uint16_t *__restrict__ P)
{
    const int64_t n = (int64_t)Epad * d;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int e = (int)(idx / d), i = (int)(idx - (int64_t)e * d);
    const float w = e < E ? W[(int64_t)i * E + e] : 0.0f;
    const uint16_t hi = f32_to_bf16(w);
    const uint16_t lo = f32_to_bf16(w - bf16_to_f32(hi));
    P[idx] = hi;
    P[n + idx] = lo;
}

constexpr int kRtTok = 128;    // tokens per block
constexpr int kRtK = 64;       // K chunk per LDS stage
constexpr int kRtStages = 4;   // LDS ring: chunks c + 1 .. c + 4 landed or in flight
constexpr int kRtMinChunks = 8;  // K chunks per block at least, when K is split

struct RouterArgs {
    const uint16_t *x;    // [T][d]
    const uint16_t *P;    // [2][Epad][d]
    const float *bias;    // [E] or null
    float *out;           // KS == 1: logits [T][E]; else partials [KS][T][E]
    int T, d, E, Epad, KS, kper;
    int ntb, net;         // token blocks (128), expert tiles (EX experts each)
};

// Router stage: [hi/lo][EX experts][8 chunks of 16 B], chunk kc of expert
// row e at slot kc ^ ((e >> 1) & 7).  Activation stage: [4 token tiles][32
// tokens][8 chunks of 16 B], chunk kc of token row t at slot kc ^ ((t >> 1) &
// 7).  Both keep the operand reads (32 rows x one chunk) free of bank
// conflicts.
constexpr int kRtXTile = 32 * 128;       // 4 KB

// EX = 64 or 32 experts per block (NT = EX / 32 expert tiles per wave).
// With 32, a batch gets twice the blocks for the same work, each re-reading
// the activations once per 32 experts instead of once per 64.
template <int EX>
__global__ __launch_bounds__(kRouterThreads) void router_gemm_kernel(RouterArgs a)
{
    constexpr int NT = EX / 32;
    constexpr int kCopies = NT + 2;        // global->LDS copies per wave and K chunk (router, activations)
    constexpr int kWStage = 2 * EX * 128;  // hi and lo rows of the block's experts, one K chunk
    constexpr int kOutRow = EX + 4;        // floats per row of an output tile in LDS (padded)
    __shared__ __attribute__((aligned(1024))) uint8_t wst[kRtStages][kWStage];
    __shared__ __attribute__((aligned(1024))) uint8_t xst[kRtStages][4][kRtXTile];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tw = wave & 3, kh = wave >> 2;  // token tile, half of each K chunk (sub-steps 2 kh, 2 kh + 1)
    const int per = a.ntb * a.net;
    const int ks = blockIdx.x / per;
    const int rem = blockIdx.x - ks * per;
    const int et = rem / a.ntb, tb = rem - et * a.ntb;
    const int n = lane & 31, h = lane >> 5;
    // router copies: copy i of wave w fills the 16-byte positions 64 (8 i + w)
    // + lane of a stage, i.e. (hi/lo, expert row, slot) = (p / (8 EX),
    // (p >> 3) % EX, p & 7); byte offsets from P at the block's first K column
    uint32_t woff[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int p = 64 * (8 * i + wave) + lane;
        const int hl = p / (8 * EX), e = (p >> 3) & (EX - 1), kc = (p & 7) ^ ((e >> 1) & 7);
        woff[i] = (uint32_t)(((size_t)hl * a.Epad + EX * et + e) * a.d * 2 + 16 * kc);
    }
    // activation copies: copy j of wave w fills rows 16 kh + 8 j + lane / 8 of
    // token tile tw, slot lane & 7; rows past T load a valid row
    uint32_t xoff[2];
    const int tok0 = kRtTok * tb + 32 * tw;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * kh + 8 * j + (lane >> 3);
        const int kc = (lane & 7) ^ ((row >> 1) & 7);
        xoff[j] = (uint32_t)min(tok0 + row, a.T - 1) * (uint32_t)a.d * 2u + 16u * (uint32_t)kc;
    }
    const int k0 = ks * a.kper, nch = a.kper / kRtK;
    auto issue = [&](int c, int stage) __attribute__((always_inline)) {
        const uint16_t *wb = a.P + k0 + c * kRtK, *xb = a.x + k0 + c * kRtK;
#pragma unroll
        for (int i = 0; i < NT; ++i) dma16(wb, woff[i], &wst[stage][(8 * i + wave) * 1024]);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(xb, xoff[j], &xst[stage][tw][(2 * kh + j) * 1024]);
    };
    f32x16 acc[NT];
#pragma unroll
    for (int v = 0; v < NT; ++v)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[v][r] = 0.f;

    // The operands of this wave's half of a chunk (per 16-wide sub-step q:
    // the activation chunk 2 q + h of token n, router chunks of experts
    // 32 v + n, hi and lo) are read from LDS into registers one chunk ahead.
    struct ChunkOps {
        bf16x8 x[2], w[2][NT][2];  // [sub-step][expert tile][hi, lo]
    };
    auto read_ops = [&](int stage, ChunkOps &o) __attribute__((always_inline)) {
        const uint8_t *ws = wst[stage], *xs = xst[stage][tw];
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int kc = 2 * (2 * kh + qq) + h;
            o.x[qq] = *reinterpret_cast<const bf16x8 *>(xs + n * 128 + 16 * (kc ^ ((n >> 1) & 7)));
#pragma unroll
            for (int v = 0; v < NT; ++v) {
                const int e = 32 * v + n;
                const int off = e * 128 + 16 * (kc ^ ((e >> 1) & 7));
                o.w[qq][v][0] = *reinterpret_cast<const bf16x8 *>(ws + off);
                o.w[qq][v][1] = *reinterpret_cast<const bf16x8 *>(ws + EX * 128 + off);
            }
        }
    };
    auto mfma_ops = [&](const ChunkOps &o) __attribute__((always_inline)) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int v = 0; v < NT; ++v) {
                acc[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[qq][v][0], o.x[qq], acc[v], 0, 0, 0);
                acc[v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[qq][v][1], o.x[qq], acc[v], 0, 0, 0);
            }
    };

    // prologue: chunks 0 .. kRtStages - 1 copied, chunk 0's operands read.
    // Every iteration issues one more chunk (clamped to the last one past
    // the end, so that the counts stay uniform).
#pragma unroll
    for (int c = 0; c < kRtStages; ++c) issue(min(c, nch - 1), c);
    ChunkOps ops[2];
    wait_vmcnt<kCopies * (kRtStages - 1)>();  // this wave's copies of chunk 0 have landed
    block_sync();                         // ... and every wave's
    read_ops(0, ops[0]);
    // Iteration c: chunk c + 1 in LDS for every wave (its copies went out
    // three iterations earlier; those of chunks c + 2 and c + 3 may be in
    // flight), then the copies of chunk c + 4 into the stage of chunk c,
    // whose operands every wave has read into registers, then the reads of
    // chunk c + 1 and the MFMAs of chunk c.
    auto iter = [&](int c, ChunkOps &cur, ChunkOps &nxt) __attribute__((always_inline)) {
        wait_vmcnt<kCopies * (kRtStages - 2)>();
        block_sync();
        issue(min(c + kRtStages, nch - 1), c % kRtStages);
        read_ops((c + 1) % kRtStages, nxt);  // past the last chunk: a stage that holds valid data
        mfma_ops(cur);
    };
    int c = 0;
    for (; c + 1 < nch; c += 2) {
        iter(c, ops[0], ops[1]);
        iter(c + 1, ops[1], ops[0]);
    }
    if (c < nch) iter(c, ops[0], ops[1]);
    wait_vmcnt<0>();  // no copy into LDS outlives the loop
    block_sync();     // ... for any wave, and every operand read is done: the stages are free

    // The two K halves of each token tile go to LDS as row-major tiles (rows
    // padded to 68 floats, so that the 16-byte writes of 16 lanes fall on
    // distinct banks): half 0 in the router stages, half 1 in the activation
    // stages.  Then every wave sums 16 rows of one tile (half 0 + half 1, in
    // that order) and stores them as whole 256-byte row segments.
    float *ot = reinterpret_cast<float *>(kh == 0 ? &wst[0][0] : &xst[0][0][0]) + tw * 32 * kOutRow;
#pragma unroll
    for (int v = 0; v < NT; ++v)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4 *>(ot + n * kOutRow + 32 * v + 8 * g + 4 * h) =
                make_float4(acc[v][4 * g], acc[v][4 * g + 1], acc[v][4 * g + 2], acc[v][4 * g + 3]);
    block_sync();
    const float *t0 = reinterpret_cast<const float *>(&wst[0][0]) + tw * 32 * kOutRow;
    const float *t1 = reinterpret_cast<const float *>(&xst[0][0][0]) + tw * 32 * kOutRow;
    const bool direct = a.KS == 1;
    constexpr int LPR = EX / 4;  // lanes per output row (4 experts each)
    const int e0 = EX * et + 4 * (lane & (LPR - 1));  // this lane's 4 experts
    float bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = (direct && a.bias && e0 + j < a.E) ? a.bias[e0 + j] : 0.f;
#pragma unroll
    for (int i = 0; i < 16 * LPR / 64; ++i) {
        const int row = 16 * kh + (64 / LPR) * i + lane / LPR;
        const int t = tok0 + row;
        if (t >= a.T) continue;
        const float4 o0 = *reinterpret_cast<const float4 *>(t0 + row * kOutRow + 4 * (lane & (LPR - 1)));
        const float4 o1 = *reinterpret_cast<const float4 *>(t1 + row * kOutRow + 4 * (lane & (LPR - 1)));
        const float val[4] = {o0.x + o1.x + bv[0], o0.y + o1.y + bv[1], o0.z + o1.z + bv[2], o0.w + o1.w + bv[3]};
        float *dst = a.out + ((size_t)ks * a.T + t) * a.E + e0;
        if ((a.E & 3) == 0) {  // rows start 16-byte aligned: all 4 experts in range or none
            if (e0 < a.E) *reinterpret_cast<float4 *>(dst) = make_float4(val[0], val[1], val[2], val[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (e0 + j < a.E) dst[j] = val[j];
        }
    }
}

// logits[t][e] = sum over the KS partials in range order (+ bias[e])
__global__ __launch_bounds__(256) void router_reduce_kernel(const float *__restrict__ part, int KS, int64_t TE,
                                                            int E, const float *__restrict__ bias,
                                                            float *__restrict__ logits)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= TE) return;
    float v = 0.f;
    for (int s = 0; s < KS; ++s) v += part[(int64_t)s * TE + idx];
    if (bias) v += bias[idx % E];
    logits[idx] = v;
}

int router_epad(int E) { return (E + 63) & ~63; }

// Experts per block: 32 where blocks of 64 would give fewer blocks than
// compute units.  Measured at T = 4096 (256 blocks of 32 against 128 of 64):
// route from x 27.7-28.5 us against 30.8-31.0 us; T = 512: 22.5 against
// 24.2-25.5 us.  At T = 32768 blocks of 32 were slower (the activations are
// read once per 32 experts instead of once per 64).
static int router_ex(int T, int E)
{
    return (int64_t)((T + kRtTok - 1) / kRtTok) * (router_epad(E) / 64) < 256 ? 32 : 64;
}

// K ranges: split until the grid has a block for every other compute unit
// (128 blocks of 8 waves), each range a whole number of K chunks and at
// least kRtMinChunks of them.  Measured at T = 4096 with 64 experts per
// block (128 blocks): no split, route from x 31.0-31.5 us, against
// 33.0-33.4 us with two K ranges (256 blocks) and their partial sum.
int router_splits(int T, int d, int E)
{
    const int64_t blocks = (int64_t)((T + kRtTok - 1) / kRtTok) * (router_epad(E) / router_ex(T, E));
    const int nch = d / kRtK;
    int ks = 1;
    while (blocks * ks < 128 && nch % (ks * 2) == 0 && nch / (ks * 2) >= kRtMinChunks) ks *= 2;
    return ks;
}

hipError_t launch_router_pack(const float *W, int d, int E, uint16_t *P, hipStream_t s)
{
    const int Epad = router_epad(E);
    const int64_t n = (int64_t)Epad * d;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(router_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, W, d, E, Epad, P);
    return hipGetLastError();
}

hipError_t launch_router(const Plan &p, const uint16_t *x, const uint16_t *P, const float *bias, float *logits,
                         void *ws, hipStream_t s)
{
    if (p.T == 0) return hipSuccess;
    RouterArgs a;
    a.x = x; a.P = P; a.bias = bias;
    a.T = p.T; a.d = p.d; a.E = p.E; a.Epad = router_epad(p.E);
    a.KS = router_splits(p.T, p.d, p.E);
    a.kper = p.d / a.KS;
    a.ntb = (p.T + kRtTok - 1) / kRtTok;
    const int ex = router_ex(p.T, p.E);
    a.net = a.Epad / ex;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_router);
    a.out = a.KS == 1 ? logits : part;
    const int64_t blocks = (int64_t)a.ntb * a.net * a.KS;
    if (ex == 32)
        hipLaunchKernelGGL(router_gemm_kernel<32>, dim3((unsigned)blocks), dim3(kRouterThreads), 0, s, a);
    else
        hipLaunchKernelGGL(router_gemm_kernel<64>, dim3((unsigned)blocks), dim3(kRouterThreads), 0, s, a);
    if (a.KS > 1) {
        const int64_t TE = (int64_t)p.T * p.E;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((TE + 255) / 256)), dim3(256), 0, s,
                           (const float *)part, a.KS, TE, p.E, bias, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
