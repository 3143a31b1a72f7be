// Decode attention of one token over grouped KV heads (gfx950): the second
// decode workload of the pages.  Eight query heads share one KV head, and
// the pages pack query heads that share a KV head into one threadgroup so
// that they share the KV loads (page "Perplexity's Lily Beats MLX-LM by 1.35x
// Running Qwen3.6 on Apple Silicon", section "Decode optimizations").  Here
// all eight query heads of a KV head live in every wave: each K and V row is
// read from HBM once and used by the eight heads in registers.
//
// o_h = sum_t softmax_t(q_h . k_{g,t} / sqrt(D)) v_{g,t}, g = h / 8, fp32
// arithmetic from bf16 inputs, bf16 output.  One token reads 2 L D bytes per
// KV head and does 8 D multiply-adds per cached token for the scores and as
// many for the output: about 4 per byte, so the step is bound by HBM, and
// the products run on the vector ALUs (v_dot2_f32_bf16 for the scores, fp32
// fma for the output) rather than being reshaped into matrix-core tiles.
//
// Kernels (stream-ordered):
//   gqa_partial_kernel<D>   grid (splits, Hkv), 4 waves: the block's C cached
//                           tokens (C a power of two, chosen so that the grid
//                           holds about 1024 blocks).  Lane l of a wave owns 8
//                           dims (8 (l % (D/8)) ..) of token l / (D/8) of an
//                           iteration of 64 / (D/8) tokens.  Pass 1: scores of
//                           the 8 heads (dot2 over the lane's dims, then a
//                           transpose-reduce over the token's lanes: 8 values
//                           halve at each exchange, so 8 exchanges instead of
//                           32 leave each lane one head's full score) into
//                           LDS; block max and exp2 weights per head.  Pass 2:
//                           o_h += p_t v_t for the lane's dims, summed over the
//                           token slots and waves at the end.  Writes the
//                           block's (max, sum, unnormalised o) per head.
//   gqa_combine_kernel      one block per query head, one thread per dim: the
//                           splits' partials rescaled to the global max and
//                           summed in split order (deterministic), o = sum /
//                           weight sum, rounded to bf16.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kAttnG = 8;          // query heads per KV head
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnUnroll = 8;     // iterations whose rows are loaded together

struct AttnArgs {
    const uint16_t *q, *k, *v;  // [Hq][D], [Hkv][L][D], [Hkv][L][D]
    int Hkv, L, C, nsplit;
    float scale2;               // log2(e) / sqrt(D)
    float *part_o;              // [nsplit][Hq][D]
    float *part_ml;             // [nsplit][Hq][2]: block max (log2 domain), weight sum
};

// Transpose-reduce of 8 per-lane partial sums over the LPT lanes of a token
// (lanes l .. l + LPT - 1 of an aligned group): at exchange distance w the
// lane keeps half of its values (the half chosen by its lane bit w) and adds
// the partner's copies of them, so the count halves at each step; after
// log2(LPT) steps every lane holds the full sum of one head, head index
// given by its low lane bits (LPT >= 8).
template <int LPT>
__device__ __forceinline__ float reduce8_over_token(float (&a)[8], int &head)
{
    const int lane = threadIdx.x & 63;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = a[i];
    int n = 8;       // live values
    int base = 0;    // head index of v[0]
#pragma unroll
    for (int w = LPT / 2; w >= 1; w >>= 1) {
        if (n > 1) {
            const bool upper = (lane & w) != 0;
            const int h = n / 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < h) {
                    // send the half the partner keeps, receive the half this lane keeps
                    const float send = upper ? v[i] : v[i + h];
                    const float keep = upper ? v[i + h] : v[i];
                    v[i] = keep + __shfl_xor(send, w);
                }
            }
            base += upper ? h : 0;
            n = h;
        } else {
            v[0] += __shfl_xor(v[0], w);
        }
    }
    head = base;
    return v[0];
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void gqa_partial_kernel(AttnArgs a)
{
    constexpr int LPT = D / 8;      // lanes per token
    constexpr int TPI = 64 / LPT;   // tokens per wave iteration
    __shared__ float s_p[kAttnThreads / 64 * 1024 / 4 * kAttnG];  // scores, then weights: [token][head]
    __shared__ float s_m[kAttnG], s_l[kAttnG], s_red[4][kAttnG];
    __shared__ float s_o[4][kAttnG][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, g = blockIdx.y;
    const int t0 = split * a.C, n = min(a.C, a.L - t0);  // tokens of the block (>= 1)
    const int per_wave = a.C / 4;                          // tokens per wave (a multiple of TPI)
    const int slot = lane / LPT, dpart = lane % LPT;       // token slot, 8-dim part
    const size_t kvbase = ((size_t)g * a.L) * D + 8 * dpart;

    // q of the 8 heads, this lane's 8 dims: 4 bf16 pairs per head
    uint32_t qr[kAttnG][4];
#pragma unroll
    for (int h = 0; h < kAttnG; ++h) {
        const uint4 u = *reinterpret_cast<const uint4 *>(a.q + (size_t)(kAttnG * g + h) * D + 8 * dpart);
        qr[h][0] = u.x; qr[h][1] = u.y; qr[h][2] = u.z; qr[h][3] = u.w;
    }

    // pass 1: scores (log2 domain) of the wave's tokens into LDS
    for (int it0 = 0; it0 < per_wave; it0 += TPI * kAttnUnroll) {
        uint4 kr[kAttnUnroll];
#pragma unroll
        for (int u = 0; u < kAttnUnroll; ++u) {
            const int tl = wave * per_wave + it0 + TPI * u + slot;  // token inside the block
            const int tt = t0 + min(tl, n - 1);                      // past the end: a valid row
            kr[u] = *reinterpret_cast<const uint4 *>(a.k + kvbase + (size_t)tt * D);
        }
#pragma unroll
        for (int u = 0; u < kAttnUnroll; ++u) {
            const int tl = wave * per_wave + it0 + TPI * u + slot;
            float part[kAttnG];
#pragma unroll
            for (int h = 0; h < kAttnG; ++h) {
                float acc = dot2_bf16(kr[u].x, qr[h][0], 0.f);
                acc = dot2_bf16(kr[u].y, qr[h][1], acc);
                acc = dot2_bf16(kr[u].z, qr[h][2], acc);
                part[h] = dot2_bf16(kr[u].w, qr[h][3], acc);
            }
            int head;
            const float s = reduce8_over_token<LPT>(part, head) * a.scale2;
            // the lanes whose bits below the three halving exchanges are 0 hold
            // the 8 heads once each
            if ((dpart & (LPT / 8 - 1)) == 0 && it0 + TPI * u < per_wave)
                s_p[tl * kAttnG + head] = tl < n ? s : -INFINITY;
        }
    }
    __syncthreads();

    // block max and weight sum per head: thread (part = tid / 8, head h =
    // tid % 8) takes tokens part, part + 32, ...; the 32 parts of a head are
    // combined over the lanes of a wave (exchanges 8, 16, 32) and then over
    // the 4 waves in order, so the sums are deterministic.  The scores
    // become the weights exp2(s - max), 0 past the block's last token.
    {
        const int h = tid & (kAttnG - 1), part = tid >> 3;
        float m = -INFINITY;
        for (int t = part; t < n; t += 32) m = fmaxf(m, s_p[t * kAttnG + h]);
        m = fmaxf(m, __shfl_xor(m, 8));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (lane < kAttnG) s_red[wave][lane] = m;
        __syncthreads();
        m = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
        float l = 0.f;
        for (int t = part; t < a.C; t += 32) {
            const float p = t < n ? exp2f(s_p[t * kAttnG + h] - m) : 0.f;
            s_p[t * kAttnG + h] = p;
            l += p;
        }
        l += __shfl_xor(l, 8);
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        __syncthreads();  // every wave has read s_red (the maxima)
        if (lane < kAttnG) s_red[wave][lane] = l;
        __syncthreads();
        if (tid < kAttnG) {
            s_m[tid] = m;
            s_l[tid] = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
        }
    }
    __syncthreads();

    // pass 2: o_h += p_t v_t over the wave's tokens, this lane's 8 dims
    float o[kAttnG][8];
#pragma unroll
    for (int h = 0; h < kAttnG; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = 0.f;
    for (int it0 = 0; it0 < per_wave; it0 += TPI * kAttnUnroll) {
        uint4 vr[kAttnUnroll];
#pragma unroll
        for (int u = 0; u < kAttnUnroll; ++u) {
            const int tl = wave * per_wave + it0 + TPI * u + slot;
            const int tt = t0 + min(tl, n - 1);
            vr[u] = *reinterpret_cast<const uint4 *>(a.v + kvbase + (size_t)tt * D);
        }
#pragma unroll
        for (int u = 0; u < kAttnUnroll; ++u) {
            if (it0 + TPI * u >= per_wave) break;
            const int tl = wave * per_wave + it0 + TPI * u + slot;
            const float4 p0 = *reinterpret_cast<const float4 *>(&s_p[tl * kAttnG]);
            const float4 p1 = *reinterpret_cast<const float4 *>(&s_p[tl * kAttnG + 4]);
            const float p[kAttnG] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};  // 0 past the end
            const uint32_t w4[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
            float vf[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vf[2 * j] = bf16_to_f32(w4[j] & 0xFFFFu);
                vf[2 * j + 1] = bf16_to_f32(w4[j] >> 16);
            }
#pragma unroll
            for (int h = 0; h < kAttnG; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) o[h][j] = __builtin_fmaf(p[h], vf[j], o[h][j]);
        }
    }
    // sum over the wave's token slots (lanes with equal dpart), then over waves
#pragma unroll
    for (int w = LPT; w < 64; w <<= 1)
#pragma unroll
        for (int h = 0; h < kAttnG; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) o[h][j] += __shfl_xor(o[h][j], w);
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < kAttnG; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) s_o[wave][h][8 * dpart + j] = o[h][j];
    }
    __syncthreads();
    const int hq0 = kAttnG * g;
    for (int i = tid; i < kAttnG * D; i += kAttnThreads) {
        const int h = i / D, dd = i - h * D;
        const float sum = ((s_o[0][h][dd] + s_o[1][h][dd]) + s_o[2][h][dd]) + s_o[3][h][dd];
        a.part_o[((size_t)split * (a.Hkv * kAttnG) + hq0 + h) * D + dd] = sum;
    }
    if (tid < kAttnG) {
        float *ml = a.part_ml + ((size_t)split * (a.Hkv * kAttnG) + hq0 + tid) * 2;
        ml[0] = s_m[tid];
        ml[1] = s_l[tid];
    }
}

// one block per query head, one thread per dim
__global__ __launch_bounds__(256) void gqa_combine_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, int Hq, int D,
                                                          int nsplit, uint16_t *__restrict__ out)
{
    const int h = blockIdx.x, i = threadIdx.x;
    if (i >= D) return;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((size_t)s * Hq + h) * 2]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float c = exp2f(part_ml[((size_t)s * Hq + h) * 2] - M);
        den += c * part_ml[((size_t)s * Hq + h) * 2 + 1];
        num += c * part_o[((size_t)s * Hq + h) * D + i];
    }
    out[(size_t)h * D + i] = f32_to_bf16(num / den);
}

// tokens per block: a power of two, 64 .. 1024, about 1024 blocks in the grid
int attn_chunk(int Hkv, int L)
{
    const int64_t want = ((int64_t)L * Hkv + 1023) / 1024;
    int c = 64;
    while (c < want && c < 1024) c <<= 1;
    return c;
}

size_t attn_workspace_bytes(int Hq, int Hkv, int D, int L)
{
    const int64_t ns = (L + attn_chunk(Hkv, L) - 1) / attn_chunk(Hkv, L);
    return (size_t)ns * Hq * (D + 2) * 4;
}

hipError_t launch_gqa_decode(int Hq, int Hkv, int D, int L, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, void *ws, hipStream_t s, EventTrace *tr)
{
    AttnArgs a;
    a.q = q; a.k = k; a.v = v;
    a.Hkv = Hkv; a.L = L;
    a.C = attn_chunk(Hkv, L);
    a.nsplit = (L + a.C - 1) / a.C;
    a.scale2 = 1.4426950408889634f / sqrtf((float)D);
    a.part_o = static_cast<float *>(ws);
    a.part_ml = a.part_o + (size_t)a.nsplit * Hq * D;
    const dim3 grid(a.nsplit, Hkv);
    switch (D) {
    case 64: launch(tr, gqa_partial_kernel<64>, grid, dim3(kAttnThreads), 0, s, a); break;
    case 128: launch(tr, gqa_partial_kernel<128>, grid, dim3(kAttnThreads), 0, s, a); break;
    default: launch(tr, gqa_partial_kernel<256>, grid, dim3(kAttnThreads), 0, s, a); break;
    }
    launch(tr, gqa_combine_kernel, dim3(Hq), dim3(256), 0, s, (const float *)a.part_o, (const float *)a.part_ml,
           Hq, D, a.nsplit, o);
    return hipGetLastError();
}

}  // namespace moe
