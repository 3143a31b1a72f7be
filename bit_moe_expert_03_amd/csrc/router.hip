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
// router_gemm_kernel: one wave = 32 tokens x 64 experts (two 32x32 tiles)
// over a K range; v_mfma_f32_32x32x16_bf16 with the weights as the first
// operand, so lane l holds token l % 32 and register r of tile u holds
// expert 64 et + 32 u + 8 (r / 4) + 4 (l / 32) + r % 4.  When the grid
// would be small (few tokens), K is split into KS ranges whose partial
// logits a second kernel sums in range order (deterministic), adding the
// bias; with KS = 1 the GEMM writes the logits itself.
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

struct RouterArgs {
    const uint16_t *x;    // [T][d]
    const uint16_t *P;    // [2][Epad][d]
    const float *bias;    // [E] or null
    float *out;           // KS == 1: logits [T][E]; else partials [KS][T][E]
    int T, d, E, Epad, KS, kper;
    int ntt, net;         // token tiles (32), expert tiles (64)
};

__global__ __launch_bounds__(kRouterThreads) void router_gemm_kernel(RouterArgs a)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kRouterThreads / kWave) + wave;
    if (gw >= a.ntt * a.net * a.KS) return;  // wave-uniform
    const int ks = gw / (a.ntt * a.net);
    const int rem = gw - ks * a.ntt * a.net;
    const int et = rem / a.ntt, tt = rem - et * a.ntt;
    const int n = lane & 31, h = lane >> 5;
    const int t = 32 * tt + n;
    const int tl = t < a.T ? t : a.T - 1;  // rows past T load a valid row; not stored
    const size_t EP = (size_t)a.Epad * a.d;
    const uint16_t *xr = a.x + (size_t)tl * a.d + 8 * h;
    const uint16_t *w0 = a.P + (size_t)(64 * et + n) * a.d + 8 * h;  // hi rows of tile 0
    const uint16_t *w1 = w0 + (size_t)32 * a.d;                       // tile 1
    f32x16 acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; }
    const int k0 = ks * a.kper, k1 = k0 + a.kper;
#pragma unroll 4
    for (int k = k0; k < k1; k += 16) {
        const bf16x8 xa = *reinterpret_cast<const bf16x8 *>(xr + k);
        const bf16x8 a0h = *reinterpret_cast<const bf16x8 *>(w0 + k);
        const bf16x8 a0l = *reinterpret_cast<const bf16x8 *>(w0 + EP + k);
        const bf16x8 a1h = *reinterpret_cast<const bf16x8 *>(w1 + k);
        const bf16x8 a1l = *reinterpret_cast<const bf16x8 *>(w1 + EP + k);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0h, xa, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1h, xa, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0l, xa, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1l, xa, acc1, 0, 0, 0);
    }
    if (t >= a.T) return;
    float *orow = a.out + ((size_t)ks * a.T + t) * a.E;
    const bool direct = a.KS == 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + 4 * h + (r & 3);
        const int e0 = 64 * et + m, e1 = e0 + 32;
        if (e0 < a.E) orow[e0] = acc0[r] + ((direct && a.bias) ? a.bias[e0] : 0.f);
        if (e1 < a.E) orow[e1] = acc1[r] + ((direct && a.bias) ? a.bias[e1] : 0.f);
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
    const int64_t waves = (int64_t)((T + 31) / 32) * (router_epad(E) / 64);
    int ks = 1;
    while (ks < 16 && waves * ks * 2 <= 1024 && (d / 16) % (ks * 2) == 0) ks *= 2;
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
    a.ntt = (p.T + 31) / 32;
    a.net = a.Epad / 64;
    float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_router);
    a.out = a.KS == 1 ? logits : part;
    const int64_t waves = (int64_t)a.ntt * a.net * a.KS;
    hipLaunchKernelGGL(router_gemm_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(kRouterThreads), 0, s, a);
    if (a.KS > 1) {
        const int64_t TE = (int64_t)p.T * p.E;
        hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((TE + 255) / 256)), dim3(256), 0, s,
                           (const float *)part, a.KS, TE, p.E, bias, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
