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
// router_gemm_kernel: one block = 256 tokens x 64 experts over a K range,
// each wave 64 tokens (two 32-token tiles) x the block's 64 experts (two
// 32-expert tiles).  The router rows of the block (hi and lo, 64 experts x
// a 64-wide K chunk, 16 KB) are staged in LDS, double-buffered, and shared
// by the four waves -- each router row is read from L2 once per 256 tokens;
// each wave loads its activation fragments from global memory one chunk
// ahead.  v_mfma_f32_32x32x16_bf16 with the router as the first operand, so
// lane l holds token l % 32 of a token tile and register r of an expert tile
// holds expert 8 (r / 4) + 4 (l / 32) + r % 4 of it.  When the grid would be
// small, K is split into KS ranges whose partial logits a second kernel sums
// in range order (deterministic), adding the bias; with KS = 1 the GEMM
// writes the logits itself.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRouterThreads = 256;  // 4 waves per block

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

constexpr int kRtTok = 256;  // tokens per block
constexpr int kRtK = 64;     // K chunk per LDS stage

struct RouterArgs {
    const uint16_t *x;    // [T][d]
    const uint16_t *P;    // [2][Epad][d]
    const float *bias;    // [E] or null
    float *out;           // KS == 1: logits [T][E]; else partials [KS][T][E]
    int T, d, E, Epad, KS, kper;
    int ntb, net;         // token blocks (256), expert tiles (64)
};

// LDS stage: [hi/lo][64 experts][64 K] bf16, the eight 16-byte chunks of
// expert row e stored at slot c ^ (e & 7) (spreads the operand reads, 32
// rows x one chunk, over the banks)
struct RtStage {
    uint4 v[2][64][8];
};

__global__ __launch_bounds__(kRouterThreads) void router_gemm_kernel(RouterArgs a)
{
    __shared__ RtStage st[2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int per = a.ntb * a.net;
    const int ks = blockIdx.x / per;
    const int rem = blockIdx.x - ks * per;
    const int et = rem / a.ntb, tb = rem - et * a.ntb;
    const int n = lane & 31, h = lane >> 5;
    const size_t EP = (size_t)a.Epad * a.d;
    // this thread's share of a stage: chunks c = tid + 256 i, i < 4, of the
    // 1024 (hi/lo, expert row, 16-byte chunk) of a stage
    const uint16_t *wsrc[4];
    int wdst_hl[4], wdst_e[4], wdst_s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int hl = c >> 9, e = (c >> 3) & 63, kc = c & 7;
        wsrc[i] = a.P + hl * EP + (size_t)(64 * et + e) * a.d + 8 * kc;
        wdst_hl[i] = hl; wdst_e[i] = e; wdst_s[i] = kc ^ (e & 7);
    }
    // this lane's activation rows (two token tiles); rows past T load a valid row
    const uint16_t *xr[2];
    int tok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        tok[u] = kRtTok * tb + 64 * wave + 32 * u + n;
        xr[u] = a.x + (size_t)min(tok[u], a.T - 1) * a.d + 8 * h;
    }
    f32x16 acc[2][2];  // [token tile][expert tile]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][v][r] = 0.f;

    const int k0 = ks * a.kper, nch = a.kper / kRtK;
    uint4 wreg[4];
    bf16x8 xa[2][2][4];  // [buffer][token tile][sub-step]
    auto load_w = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[i] = *reinterpret_cast<const uint4 *>(wsrc[i] + kc);
    };
    auto store_w = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[b].v[wdst_hl[i]][wdst_e[i]][wdst_s[i]] = wreg[i];
    };
    auto load_x = [&](int b, int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) xa[b][u][q] = *reinterpret_cast<const bf16x8 *>(xr[u] + kc + 16 * q);
    };
    load_w(k0);
    load_x(0, k0);
    store_w(0);
    __syncthreads();
    // chunk c computes from stage c % 2 and activation buffer c % 2 while the
    // next chunk's router rows and activations are loaded
    auto chunk = [&](auto bc, int c) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        const bool more = c + 1 < nch;
        if (more) {
            load_w(k0 + (c + 1) * kRtK);
            load_x(b ^ 1, k0 + (c + 1) * kRtK);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // 16-wide sub-steps of the chunk
            const int slot_h = 2 * q + h;
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int e = 32 * v + n;
                const bf16x8 wh = __builtin_bit_cast(bf16x8, st[b].v[0][e][slot_h ^ (e & 7)]);
                const bf16x8 wlo = __builtin_bit_cast(bf16x8, st[b].v[1][e][slot_h ^ (e & 7)]);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, xa[b][u][q], acc[u][v], 0, 0, 0);
                    acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wlo, xa[b][u][q], acc[u][v], 0, 0, 0);
                }
            }
        }
        if (more) store_w(b ^ 1);  // stage b ^ 1 was last read before the previous barrier
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
        chunk(std::integral_constant<int, 0>(), c);
        if (c + 1 < nch) chunk(std::integral_constant<int, 1>(), c + 1);
    }
    const bool direct = a.KS == 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (tok[u] >= a.T) continue;
        float *orow = a.out + ((size_t)ks * a.T + tok[u]) * a.E;
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = 64 * et + 32 * v + 8 * (r >> 2) + 4 * h + (r & 3);
                if (e < a.E) orow[e] = acc[u][v][r] + ((direct && a.bias) ? a.bias[e] : 0.f);
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

// K ranges: enough waves to spread a small batch over the chip (about 1024),
// each range a whole number of 16-wide K steps
int router_splits(int T, int d, int E)
{
    const int64_t blocks = (int64_t)((T + kRtTok - 1) / kRtTok) * (router_epad(E) / 64);
    int ks = 1;
    while (ks < 16 && blocks * ks * 2 <= 512 && (d / kRtK) % (ks * 2) == 0) ks *= 2;
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
    a.net = a.Epad / 64;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_router);
    a.out = a.KS == 1 ? logits : part;
    const int64_t blocks = (int64_t)a.ntb * a.net * a.KS;
    hipLaunchKernelGGL(router_gemm_kernel, dim3((unsigned)blocks), dim3(kRouterThreads), 0, s, a);
    if (a.KS > 1) {
        const int64_t TE = (int64_t)p.T * p.E;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((TE + 255) / 256)), dim3(256), 0, s,
                           (const float *)part, a.KS, TE, p.E, bias, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
