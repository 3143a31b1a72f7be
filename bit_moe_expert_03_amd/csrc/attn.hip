// Decode attention of one token over grouped KV heads (gfx950): the second
// decode workload of the pages.  Eight query heads share one KV head, and
// the pages pack four of them into one threadgroup so that they share the
// KV loads (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on
// Apple Silicon", section "Decode optimizations").  Here all eight query
// heads of a KV head are the columns of one matrix-core tile: each K and V
// row is read from HBM once and used by all eight heads.
//
// o_h = sum_t softmax_t(q_h . k_{g,t} / sqrt(D)) v_{g,t}, g = h / 8, bf16
// inputs, fp32 accumulation, bf16 output.  One token reads 2 L D bytes per
// KV head, so the step is bound by HBM.  On the vector ALUs the products
// would cost about as many cycles as the bytes take to arrive (8 heads x 2
// products per bf16 element), so the two contractions run on the matrix
// cores, with the eight heads padded to a 16-wide tile:
//   scores  S^T = K Q^T     v_mfma_f32_16x16x32_bf16: rows = 16 tokens,
//                           columns = heads, K = head dims (bf16 products
//                           are exact in fp32);
//   output  O^T = V^T P^T   rows = 16 head dims, columns = heads, K = the
//                           slice's 32 tokens (v_mfma_f32_16x16x32_bf16) or
//                           16 (v_mfma_f32_16x16x16_bf16).  P is split into
//                           bf16 hi + lo parts (two MFMAs), which keeps about
//                           16 bits of each weight, so the output carries
//                           fp32-level error.
// The score tile leaves lane l with head l % 16 and tokens 4 (l / 16) + i,
// which is exactly a B operand of the output MFMA once the tokens of the
// slice's score tiles are ordered tau(g, k) = 16 (k / 4) + 4 g + k % 4: the
// weights never leave the lane.  V^T is formed in registers: lane (r, g)
// loads dims D/16 r .. of its tokens tau(g, .) and interleaves them pairwise
// (one byte permute per output word), so every A operand is one
// token-contiguous column of V; row r of output tile n is head dim (D/16) r + n.
//
// Kernels (stream-ordered):
//   gqa_partial_kernel<D, NJ>  grid (splits, Hkv), 4 waves, one round of
//                           blocks (blocks per CU from the occupancy of the
//                           kernel times the CUs); a block takes C consecutive
//                           tokens, its waves take interleaved slices of
//                           16 NJ tokens (NJ = 2; NJ = 1 where a context is
//                           too short to fill the grid otherwise), each with
//                           its own online softmax (running max per head,
//                           rescale of the accumulators when it grows), so
//                           the main loop has no block barrier.  The four
//                           waves are merged through LDS; writes the block's
//                           (max, weight sum, unnormalised o) per query head.
//   gqa_combine_kernel      grid (Hq, D/16): the splits' partials rescaled to
//                           the global max and summed in a fixed order
//                           (deterministic), o = sum / weight sum, bf16.
#include "moe_device.h"
#include "moe_internal.h"

#include <atomic>

namespace moe {

constexpr int kAttnG = 8;            // query heads per KV head
constexpr int kAttnThreads = 256;    // 4 waves
constexpr int kAttnMaxSplits = 1024;
constexpr int kAttnCombineThreads = 256;

struct AttnArgs {
    const uint16_t *q, *k, *v;  // [Hq][D], [Hkv][L][D], [Hkv][L][D]
    int Hkv, L, C, nsplit;
    float scale2;               // log2(e) / sqrt(D)
    float *part_o;              // [nsplit][Hq][D]
    float *part_ml;             // [nsplit][Hq][2]: block max (log2 domain), weight sum
};

// K and V rows are read once per call: non-temporal loads (nt bit), so the
// stream does not displace the caches' other contents
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream4(const uint16_t *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_stream2(const uint16_t *p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v[0], v[1]);
}

// 2^x by the hardware instruction alone: no rescaling for results below
// 2^-126, which come out as 0.  For softmax weights (x <= 0 against the
// running max) that drops only weights under 2^-126 of the largest one.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: the same lane layout with 4 contraction slots per lane
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16k16(uint2 a, uint2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                     c, 0, 0, 0);
}

// NJ: 16-token score tiles per wave slice (slices of 16 NJ tokens; the
// output MFMA contracts over the slice: 16x16x32 for NJ = 2, 16x16x16 for
// NJ = 1, which short contexts take to put twice as many waves to work)
template <int D, int NJ>
__global__ __launch_bounds__(kAttnThreads, 2) void gqa_partial_kernel(AttnArgs a)
{
    constexpr int SL = 16 * NJ;  // tokens per wave slice
    constexpr int TL = 4 * NJ;   // tokens per lane in the output MFMA's K block
    constexpr int PW = 2 * NJ;   // words per lane of a weight operand
    constexpr int DPL = D / 16;  // head dims per lane in the output tiles (= number of tiles)
    constexpr int VW = DPL / 2;  // words of V per lane and token
    constexpr int KK = D / 32;   // score MFMAs per 16-token tile
    __shared__ float s_o[4][kAttnG][D];
    __shared__ float s_m[4][kAttnG], s_l[4][kAttnG];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, g = blockIdx.y;
    const int t0 = split * a.C, n = min(a.C, a.L - t0);  // tokens of the block (>= 1)
    const uint16_t *kb = a.k + ((size_t)g * a.L + t0) * D;
    const uint16_t *vb = a.v + ((size_t)g * a.L + t0) * D;
    const bool head_ok = r < kAttnG;  // columns 8..15 of the tiles are padding

    // B operand of the scores: column r = query head 8 g + r, K chunk kk =
    // dims 32 kk + 8 grp .. + 7 (the A operand takes the same dims)
    uint4 qb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qb[kk] = head_ok ? *reinterpret_cast<const uint4 *>(a.q + (size_t)(kAttnG * g + r) * D + 32 * kk + 8 * grp)
                         : make_uint4(0, 0, 0, 0);

    f32x4 oacc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // K rows of the NJ 16-token tiles of a slice (row r of tile j = token
    // base + 16 j + r); past the block's last token, the last valid row is
    // read and its score masked.  Up to D = 128 the next slice's K rows are
    // loaded into the same registers as soon as the score MFMAs have read
    // them, so they arrive under this slice's softmax and output work (at
    // D = 256 that would not fit the registers of two blocks per CU).
    constexpr bool kPrefetchK = D <= 128;
    uint4 kr[NJ][KK];
    auto load_k = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int t = min(base + 16 * j + r, n - 1);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                kr[j][kk] = load_stream4(kb + (size_t)t * D + 32 * kk + 8 * grp);
        }
    };
    if (kPrefetchK && SL * wave < n) load_k(SL * wave);
    for (int base = SL * wave; base < n; base += 4 * SL) {
        if (!kPrefetchK) load_k(base);
        // V of tokens tau(grp, k), dims DPL r .. DPL r + DPL - 1
        uint32_t vw[TL][VW];
#pragma unroll
        for (int k = 0; k < TL; ++k) {
            const int t = min(base + 16 * (k >> 2) + 4 * grp + (k & 3), n - 1);
            const uint16_t *src = vb + (size_t)t * D + DPL * r;
            if constexpr (VW == 2) {
                const uint2 u = load_stream2(src);
                vw[k][0] = u.x; vw[k][1] = u.y;
            } else {
#pragma unroll
                for (int c = 0; c < VW / 4; ++c) {
                    const uint4 u = load_stream4(src + 8 * c);
                    vw[k][4 * c] = u.x; vw[k][4 * c + 1] = u.y; vw[k][4 * c + 2] = u.z; vw[k][4 * c + 3] = u.w;
                }
            }
        }

        // scores: lane holds head r, tokens base + 16 j + 4 grp + i
        f32x4 sc[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) sc[j] = mfma16(kr[j][kk], qb[kk], sc[j]);
        }
        if (kPrefetchK && base + 4 * SL < n) load_k(base + 4 * SL);
        float s[TL];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < TL; ++k) {
            const int t = base + 16 * (k >> 2) + 4 * grp + (k & 3);
            s[k] = (head_ok && t < n) ? sc[k >> 2][k & 3] * a.scale2 : -INFINITY;
            mx = fmaxf(mx, s[k]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == m_run ? 1.f : exp2_fast(m_run - m_new);  // 1 while nothing is valid
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < DPL; ++i) oacc[i] *= alpha;
            l_run *= alpha;
        }
        m_run = m_new;

        // weights and their bf16 hi / lo parts: B operand of the output MFMAs
        // (K position k = token tau(grp, k))
        uint32_t ph[PW], pl[PW];
#pragma unroll
        for (int w = 0; w < PW; ++w) {
            const float p0 = s[2 * w] == -INFINITY ? 0.f : exp2_fast(s[2 * w] - m_new);
            const float p1 = s[2 * w + 1] == -INFINITY ? 0.f : exp2_fast(s[2 * w + 1] - m_new);
            l_run += p0 + p1;
            ph[w] = pack_bf16x2(p0, p1);
            pl[w] = pack_bf16x2(p0 - __uint_as_float(ph[w] << 16), p1 - __uint_as_float(ph[w] & 0xFFFF0000u));
        }
        // output tiles: A operand of tile nt = dim DPL r + nt of tokens tau(grp, 0..TL-1)
#pragma unroll
        for (int nt = 0; nt < DPL; ++nt) {
            uint32_t av[PW];
#pragma unroll
            for (int w = 0; w < PW; ++w) {
                const uint32_t x = vw[2 * w][nt >> 1], y = vw[2 * w + 1][nt >> 1];
                // (low halves of x, y) or (high halves of x, y): one byte permute
                av[w] = (nt & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
            }
            if constexpr (NJ == 2) {
                const uint4 au = make_uint4(av[0], av[1], av[2], av[3]);
                oacc[nt] = mfma16(au, make_uint4(ph[0], ph[1], ph[2], ph[3]), oacc[nt]);
                oacc[nt] = mfma16(au, make_uint4(pl[0], pl[1], pl[2], pl[3]), oacc[nt]);
            } else {
                const uint2 au = make_uint2(av[0], av[1]);
                oacc[nt] = mfma16k16(au, make_uint2(ph[0], ph[1]), oacc[nt]);
                oacc[nt] = mfma16k16(au, make_uint2(pl[0], pl[1]), oacc[nt]);
            }
        }
    }

    // merge the waves: lane (r, grp) holds o[head r][DPL (4 grp + i) + nt]
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (head_ok) {
#pragma unroll
        for (int nt = 0; nt < DPL; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_o[wave][r][DPL * (4 * grp + i) + nt] = oacc[nt][i];
        if (grp == 0) {
            s_m[wave][r] = m_run;
            s_l[wave][r] = l_run;
        }
    }
    __syncthreads();
    const int hq0 = kAttnG * g, Hq = kAttnG * a.Hkv;
    for (int i = tid; i < kAttnG * D; i += kAttnThreads) {
        const int h = i / D, dd = i - h * D;
        const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));  // finite
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float c = s_m[w][h] == -INFINITY ? 0.f : exp2_fast(s_m[w][h] - M);
            o += c * s_o[w][h][dd];
            l += c * s_l[w][h];
        }
        a.part_o[((size_t)split * Hq + hq0 + h) * D + dd] = o;
        if (dd == 0) {
            float *ml = a.part_ml + ((size_t)split * Hq + hq0 + h) * 2;
            ml[0] = M;
            ml[1] = l;
        }
    }
}

// grid (Hq, D / 16): thread (j, d) sums splits j, j + 16, ... of dim d of
// block.y's 16 dims; the 16 sums are added in order.  Every global load
// (the splits' max and weight sum, and up to 16 partial outputs per thread)
// is issued before the first reduction, so the kernel waits on memory about
// once.
constexpr int kCombinePerThread = 16;

__global__ __launch_bounds__(kAttnCombineThreads) void gqa_combine_kernel(const float *__restrict__ part_o,
                                                                          const float *__restrict__ part_ml, int Hq,
                                                                          int D, int nsplit,
                                                                          uint16_t *__restrict__ out)
{
    constexpr int kML = kAttnMaxSplits / kAttnCombineThreads;  // (max, sum) pairs per thread
    __shared__ float s_c[kAttnMaxSplits];
    __shared__ float s_red[2][4];
    __shared__ float s_num[16][17];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = tid >> 4, dl = tid & 15, d = 16 * blockIdx.y + dl;

    float2 ml[kML];
#pragma unroll
    for (int i = 0; i < kML; ++i) {
        const int s = tid + kAttnCombineThreads * i;
        ml[i] = s < nsplit ? *reinterpret_cast<const float2 *>(part_ml + ((size_t)s * Hq + h) * 2)
                           : make_float2(-INFINITY, 0.f);
    }
    float po[kCombinePerThread];
#pragma unroll
    for (int i = 0; i < kCombinePerThread; ++i) {
        const int s = j + 16 * i;
        po[i] = s < nsplit ? part_o[((size_t)s * Hq + h) * D + d] : 0.f;
    }

    float m = ml[0].x;
#pragma unroll
    for (int i = 1; i < kML; ++i) m = fmaxf(m, ml[i].x);
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) m = fmaxf(m, __shfl_xor(m, w));
    if (lane == 0) s_red[0][wave] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));  // finite

    float den = 0.f;
#pragma unroll
    for (int i = 0; i < kML; ++i) {
        const int s = tid + kAttnCombineThreads * i;
        if (s < nsplit) {
            const float c = exp2f(ml[i].x - M);
            s_c[s] = c;
            den += c * ml[i].y;
        }
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) den += __shfl_xor(den, w);
    if (lane == 0) s_red[1][wave] = den;
    __syncthreads();
    den = ((s_red[1][0] + s_red[1][1]) + s_red[1][2]) + s_red[1][3];

    float num = 0.f;
#pragma unroll
    for (int i = 0; i < kCombinePerThread; ++i) {
        const int s = j + 16 * i;
        if (s < nsplit) num += s_c[s] * po[i];
    }
    for (int s = j + 16 * kCombinePerThread; s < nsplit; s += 16)  // more than 256 splits
        num += s_c[s] * part_o[((size_t)s * Hq + h) * D + d];
    s_num[j][dl] = num;
    __syncthreads();
    if (tid < 16) {
        float t = 0.f;
        for (int i = 0; i < 16; ++i) t += s_num[i][tid];
        out[(size_t)h * D + 16 * blockIdx.y + tid] = f32_to_bf16(t / den);
    }
}

// Splits per KV head: at most kAttnMaxSplits and at most one per 64 tokens.
static int attn_max_splits(int L)
{
    return (int)std::min<int64_t>(kAttnMaxSplits, ((int64_t)L + 63) / 64);
}

size_t attn_workspace_bytes(int Hq, int Hkv, int D, int L)
{
    (void)Hkv;
    return (size_t)attn_max_splits(L) * Hq * (D + 2) * 4;
}

// Blocks of gqa_partial_kernel<D, NJ> that the device runs at once
// (occupancy per CU times CUs), queried once per device and variant.
template <int D, int NJ>
static int attn_resident_blocks()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gqa_partial_kernel<D, NJ>, kAttnThreads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

int attn_chunk(int Hkv, int L, int resident, int round)
{
    const int want = std::max(1, std::min(attn_max_splits(L), (resident + Hkv - 1) / Hkv));
    const int64_t per = ((int64_t)L + want - 1) / want;
    // A split that is not a multiple of a round (the block's four slices)
    // leaves its waves one slice apart.  Long splits (512 tokens and more)
    // take that for a grid that fills the device more closely (L = 131072:
    // 748 blocks instead of 684, 6.0 against 5.7 TB/s); short ones keep
    // whole rounds (L = 32768, 2 slices per wave: 14.4 against 15.2 us).
    const int64_t quantum = per >= 512 ? 32 : round;
    return (int)std::max<int64_t>(round, (per + quantum - 1) / quantum * quantum);
}

template <int D>
static void launch_partial(EventTrace *tr, int nj, dim3 grid, hipStream_t s, const AttnArgs &a)
{
    if (nj == 1)
        launch(tr, gqa_partial_kernel<D, 1>, grid, dim3(kAttnThreads), 0, s, a);
    else
        launch(tr, gqa_partial_kernel<D, 2>, grid, dim3(kAttnThreads), 0, s, a);
}

template <int D>
static int attn_plan(int Hkv, int L, int *nj)
{
    // 32-token slices; where that gives each wave a single slice and leaves
    // the grid short of the co-resident block count (short contexts), 16-token
    // slices put twice as many waves to work, each with half the arithmetic
    const int resident2 = attn_resident_blocks<D, 2>();
    const int c2 = attn_chunk(Hkv, L, resident2, 128);
    if (c2 == 128 && (int64_t)((L + 127) / 128) * Hkv < resident2) {
        *nj = 1;
        return attn_chunk(Hkv, L, attn_resident_blocks<D, 1>(), 64);
    }
    *nj = 2;
    return c2;
}

hipError_t launch_gqa_decode(int Hq, int Hkv, int D, int L, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, void *ws, hipStream_t s, EventTrace *tr)
{
    int nj = 2;
    AttnArgs a;
    a.q = q; a.k = k; a.v = v;
    a.Hkv = Hkv; a.L = L;
    a.C = D == 64 ? attn_plan<64>(Hkv, L, &nj) : D == 128 ? attn_plan<128>(Hkv, L, &nj) : attn_plan<256>(Hkv, L, &nj);
    a.nsplit = (L + a.C - 1) / a.C;  // <= attn_max_splits(L), since C >= max(64, L / max splits)
    a.scale2 = 1.4426950408889634f / sqrtf((float)D);
    a.part_o = static_cast<float *>(ws);
    a.part_ml = a.part_o + (size_t)a.nsplit * Hq * D;
    const dim3 grid(a.nsplit, Hkv);
    switch (D) {
    case 64: launch_partial<64>(tr, nj, grid, s, a); break;
    case 128: launch_partial<128>(tr, nj, grid, s, a); break;
    default: launch_partial<256>(tr, nj, grid, s, a); break;
    }
    launch(tr, gqa_combine_kernel, dim3(Hq, D / 16), dim3(kAttnCombineThreads), 0, s, (const float *)a.part_o,
           (const float *)a.part_ml, Hq, D, a.nsplit, o);
    return hipGetLastError();
}

}  // namespace moe
