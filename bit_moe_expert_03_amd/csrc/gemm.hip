// Prefill path of the MoE layer (gfx950): grouped GEMMs over the tile block
// map, with the groupwise affine 4-bit weights decoded inside the kernel.
//
// The Lily pages unpack one 4-bit tile at a time into threadgroup memory
// right before the multiply and never write a bf16 copy of the weights
// (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
// Silicon", section "Prefill optimizations", first bullet), and treat prefill
// as a compute-bound matrix problem because every weight block serves many
// token rows (section "Why prefill and decode get different treatment").
// On CDNA4 the decode goes one step further: each lane loads the 16 bytes of
// codes it owns in the matrix-core operand layout straight into registers,
// decodes them there (fp32 fma, then a round-to-nearest-even pack to bf16)
// and feeds v_mfma_f32_32x32x16_bf16 -- the bf16 weights never exist outside
// the registers of one wave, and each weight is decoded once per block.
// The activations (gathered token rows) are staged through a 3-deep LDS ring
// (every wave of the block reads all of them); A loads are issued two steps
// ahead through registers, B codes two steps ahead, so HBM latency hides
// behind two steps of matrix-core work.
//
// Kernels (stream-ordered, no host round trip):
//   moe_gateup_kernel   routed tiles (rows gathered through perm) and shared
//                       tiles (token rows) in one grid:
//                       h = bf16(silu(A W_gate^T) * (A W_up^T))
//   moe_down_kernel     routed and shared tiles in one grid:
//                       o = w_route * (h W_down^T) -> bf16 rows: routed rows
//                       in sorted order, then the T shared rows (weight 1)
//   moe_combine_kernel  y[t] = bf16(sum_j o[inv_perm[t k + j]] + o[T k + t]),
//                       slot order then shared, fp32: deterministic, no
//                       atomics.
//
// MFMA 32x32x16 operand layout used (wave64): lane l holds row (A) or
// column (B) l % 32 and the 8 contraction slots of half h = l / 32; the
// contraction index of slot j in sub-step s of a 64-wide K step is
// k = 32 h + 8 s + j for BOTH operands (any common assignment is valid),
// which makes each lane's B codes one contiguous 16-byte load and its A
// operand one contiguous 16-byte LDS read.  Accumulator register r of lane l
// is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kGemmThreads = 256;      // 4 waves
constexpr int kKStep = 64;             // contraction per main-loop step
constexpr int kLdsPitch = kKStep + 8;  // bf16 per LDS row (pad against bank conflicts)
constexpr int kStages = 3;             // LDS ring depth for A

struct GemmTiles {
    const int32_t *tile_expert, *tile_row0, *tile_rows, *num_tiles;
    int max_tiles;
};

struct GateUpArgs {
    const uint16_t *x;      // [T][d]
    const int32_t *perm;    // [T*k]
    int T, d, k, G, F, Fs;
    moe_qmat gate, up, sgate, sup;
    GemmTiles tiles;
    int ntn_r, ntn_s;       // 128-column blocks per tile (routed, shared)
    int nblk_r, nblk_s;     // blocks of the routed and the shared part
    int nblk_pad;           // grid size (multiple of 8)
    uint16_t *h_r;          // [T*k][F] sorted rows
    uint16_t *h_s;          // [T][Fs]
};

struct DownArgs {
    const uint16_t *h_r, *h_s;
    const int32_t *perm;
    const float *topk_w;
    int T, d, k, G, F, Fs;
    moe_qmat down, sdown;
    GemmTiles tiles;
    int ntn;                // 256-column blocks (d / 256, rounded up)
    int nblk_r, nblk_s, nblk_pad;
    uint16_t *obuf;         // [T*k + T][d] weighted outputs: sorted routed rows, then shared
};

// Blocks are dispatched round-robin over the 8 XCDs; renumber them so that
// consecutive logical blocks (the column blocks of one tile, then the next
// tile of the same expert) run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk_pad)
{
    const int per = nblk_pad >> 3;
    return (bid & 7) * per + (bid >> 3);
}

template <int BM>
struct ATile {
    static constexpr int kPer = BM * (kKStep / 8) / kGemmThreads;  // 16-byte chunks per thread
    uint4 v[kPer];
};

template <int BM>
__device__ __forceinline__ void a_load(ATile<BM> &t, const uint16_t *const (&rowp)[ATile<BM>::kPer],
                                       int kcol0)
{
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < ATile<BM>::kPer; ++i)
        t.v[i] = rowp[i] ? *reinterpret_cast<const uint4 *>(rowp[i] + kcol0 + chunk * 8)
                         : make_uint4(0, 0, 0, 0);
}

template <int BM>
__device__ __forceinline__ void a_store(const ATile<BM> &t, uint16_t *lds)
{
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < ATile<BM>::kPer; ++i) {
        const int row = (threadIdx.x >> 3) + i * (kGemmThreads / 8);
        *reinterpret_cast<uint4 *>(lds + row * kLdsPitch + chunk * 8) = t.v[i];
    }
}

// B operand source of one lane: a row of a packed matrix
struct BRow {
    const uint8_t *q;   // codes of the row
    const uint16_t *s;  // scales of the row
    const uint16_t *b;  // biases of the row
};

struct BRaw {
    uint4 q;
    uint32_t sb;  // bf16 scale (low half), bf16 bias (high half)
};

__device__ __forceinline__ void b_load(BRaw &r, const BRow &row, int kstep, int half, int G)
{
    const int k0 = kstep * kKStep + 32 * half;
    r.q = *reinterpret_cast<const uint4 *>(row.q + (k0 >> 1));
    const int g = k0 / G;
    r.sb = (uint32_t)row.s[g] | ((uint32_t)row.b[g] << 16);
}

__device__ __forceinline__ void b_decode(const BRaw &r, bf16x8 op[4])
{
    const float s = __uint_as_float(r.sb << 16), b = __uint_as_float(r.sb & 0xFFFF0000u);
    const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t o[4];
        dequant8_bf16(w[i], s, b, o);
        op[i] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

// Main loop shared by both GEMMs: acc0 += A B0^T, acc1 += A B1^T over K for
// the BM rows of the tile (32-row sub-tiles past `rows` are skipped).
template <int BM>
__device__ __forceinline__ void mainloop(const uint16_t *const (&rowp)[ATile<BM>::kPer], int K,
                                         const BRow &b0, const BRow &b1, bool wave_active, int G,
                                         int rows, uint16_t *lds, f32x16 (&acc0)[BM / 32],
                                         f32x16 (&acc1)[BM / 32])
{
    constexpr int MS = BM / 32;
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, r32 = lane & 31;
    const int nk = K / kKStep;
    const int msub = (rows + 31) >> 5;  // sub-tiles with live rows (block-uniform)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { acc0[i][r] = 0.f; acc1[i][r] = 0.f; }

    // prologue: A step 0 in LDS, A step 1 in registers, B steps 0 and 1 in registers
    ATile<BM> at;
    BRaw bq[2][2];
    a_load<BM>(at, rowp, 0);
    if (wave_active) {
        b_load(bq[0][0], b0, 0, half, G);
        b_load(bq[0][1], b1, 0, half, G);
        if (nk > 1) { b_load(bq[1][0], b0, 1, half, G); b_load(bq[1][1], b1, 1, half, G); }
    }
    a_store<BM>(at, lds);
    if (nk > 1) a_load<BM>(at, rowp, kKStep);

    auto step = [&](int kt, BRaw (&cur)[2]) {
        // stage the A tile of step kt+1 (loaded one step ago), fetch kt+2
        if (kt + 1 < nk) a_store<BM>(at, lds + ((kt + 1) % kStages) * (BM * kLdsPitch));
        if (kt + 2 < nk) a_load<BM>(at, rowp, (kt + 2) * kKStep);
        __syncthreads();
        if (!wave_active) return;
        bf16x8 op0[4], op1[4];
        b_decode(cur[0], op0);
        b_decode(cur[1], op1);
        if (kt + 2 < nk) { b_load(cur[0], b0, kt + 2, half, G); b_load(cur[1], b1, kt + 2, half, G); }
        const uint16_t *buf = lds + (kt % kStages) * (BM * kLdsPitch);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                if (i < msub) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        buf + (32 * i + r32) * kLdsPitch + 32 * half + 8 * s);
                    acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op0[s], acc0[i], 0, 0, 0);
                    acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op1[s], acc1[i], 0, 0, 0);
                }
            }
        }
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, bq[0]);
        if (kt + 1 < nk) step(kt + 1, bq[1]);
    }
}

template <int BM>
__global__ __launch_bounds__(kGemmThreads, 2) void moe_gateup_kernel(GateUpArgs a)
{
    constexpr int MS = BM / 32;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kStages * BM * kLdsPitch];
    const int L = xcd_logical_block(blockIdx.x, a.nblk_pad);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int row0, rows, N, nt;
    const moe_qmat *mg, *mu;
    size_t ebase;  // first row of the expert's slab
    uint16_t *out;
    bool routed;
    if (L < a.nblk_r) {
        const int tile = L / a.ntn_r;
        nt = L - tile * a.ntn_r;
        if (tile >= *a.tiles.num_tiles) return;
        const int e = a.tiles.tile_expert[tile];
        row0 = a.tiles.tile_row0[tile];
        rows = a.tiles.tile_rows[tile];
        N = a.F; mg = &a.gate; mu = &a.up;
        ebase = (size_t)e * a.F;
        out = a.h_r;
        routed = true;
    } else if (L < a.nblk_r + a.nblk_s) {
        const int tile = (L - a.nblk_r) / a.ntn_s;
        nt = (L - a.nblk_r) - tile * a.ntn_s;
        row0 = tile * BM;
        rows = min(BM, a.T - row0);
        N = a.Fs; mg = &a.sgate; mu = &a.sup;
        ebase = 0;
        out = a.h_s;
        routed = false;
    } else {
        return;
    }
    // gathered A rows owned by this thread for the global->LDS copy
    const uint16_t *rowp[ATile<BM>::kPer];
#pragma unroll
    for (int i = 0; i < ATile<BM>::kPer; ++i) {
        const int m = (threadIdx.x >> 3) + i * (kGemmThreads / 8);
        if (m < rows) {
            const int tok = routed ? a.perm[row0 + m] / a.k : row0 + m;
            rowp[i] = a.x + (size_t)tok * a.d;
        } else {
            rowp[i] = nullptr;
        }
    }
    const int ncol0 = nt * 128 + 32 * wave;  // first h column of this wave
    const bool wave_active = ncol0 < N;
    const int n = ncol0 + (lane & 31);
    const size_t brow = ebase + (wave_active ? n : 0);
    const int Kq = a.d >> 1, Kg = a.d / a.G;
    BRow b0 = {mg->q + brow * Kq, mg->s + brow * Kg, mg->b + brow * Kg};
    BRow b1 = {mu->q + brow * Kq, mu->s + brow * Kg, mu->b + brow * Kg};
    f32x16 accg[MS], accu[MS];
    mainloop<BM>(rowp, a.d, b0, b1, wave_active, a.G, rows, lds, accg, accu);
    if (!wave_active) return;
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
            if (m < rows)
                out[(size_t)(row0 + m) * N + n] = f32_to_bf16(silu(accg[i][r]) * accu[i][r]);
        }
}

template <int BM>
__global__ __launch_bounds__(kGemmThreads, 2) void moe_down_kernel(DownArgs a)
{
    constexpr int MS = BM / 32;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kStages * BM * kLdsPitch];
    const int L = xcd_logical_block(blockIdx.x, a.nblk_pad);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int row0, rows, K, nt;
    const moe_qmat *m;
    size_t ebase;
    const uint16_t *hsrc;
    int orow0;  // first output row in obuf
    bool routed;
    if (L < a.nblk_r) {
        const int tile = L / a.ntn;
        nt = L - tile * a.ntn;
        if (tile >= *a.tiles.num_tiles) return;
        ebase = (size_t)a.tiles.tile_expert[tile] * a.d;
        row0 = a.tiles.tile_row0[tile];
        rows = a.tiles.tile_rows[tile];
        K = a.F; m = &a.down; hsrc = a.h_r;
        orow0 = row0;
        routed = true;
    } else if (L < a.nblk_r + a.nblk_s) {
        const int tile = (L - a.nblk_r) / a.ntn;
        nt = (L - a.nblk_r) - tile * a.ntn;
        row0 = tile * BM;
        rows = min(BM, a.T - row0);
        ebase = 0;
        K = a.Fs; m = &a.sdown; hsrc = a.h_s;
        orow0 = a.T * a.k + row0;
        routed = false;
    } else {
        return;
    }
    const uint16_t *rowp[ATile<BM>::kPer];
#pragma unroll
    for (int i = 0; i < ATile<BM>::kPer; ++i) {
        const int mm = (threadIdx.x >> 3) + i * (kGemmThreads / 8);
        rowp[i] = (mm < rows) ? hsrc + (size_t)(row0 + mm) * K : nullptr;
    }
    const int ncol0 = nt * 256 + 64 * wave;  // this wave: columns [ncol0, ncol0 + 64)
    const bool wave_active = ncol0 < a.d;
    const int n = ncol0 + (lane & 31);
    const int Kq = K >> 1, Kg = K / a.G;
    const size_t r0 = ebase + (wave_active ? n : 0), r1 = r0 + (wave_active ? 32 : 0);
    BRow b0 = {m->q + r0 * Kq, m->s + r0 * Kg, m->b + r0 * Kg};
    BRow b1 = {m->q + r1 * Kq, m->s + r1 * Kg, m->b + r1 * Kg};
    f32x16 acc0[MS], acc1[MS];
    mainloop<BM>(rowp, K, b0, b1, wave_active, a.G, rows, lds, acc0, acc1);
    if (!wave_active) return;
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mm = 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
            if (mm >= rows) continue;
            const float wr = routed ? a.topk_w[a.perm[row0 + mm]] : 1.0f;
            uint16_t *o = a.obuf + (size_t)(orow0 + mm) * a.d;
            o[n] = f32_to_bf16(wr * acc0[i][r]);
            o[n + 32] = f32_to_bf16(wr * acc1[i][r]);
        }
}

// one wave per token: 16-byte loads of the k routed rows and the shared row
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ obuf,
                                                          const int32_t *__restrict__ inv_perm,
                                                          int T, int k, int d,
                                                          uint16_t *__restrict__ y)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const int64_t shared_row = (int64_t)T * k + t;
    for (int c = lane * 8; c < d; c += 64 * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j <= k; ++j) {
            const int64_t row = (j < k) ? (int64_t)inv_perm[(int64_t)t * k + j] : shared_row;
            const uint4 v = *reinterpret_cast<const uint4 *>(obuf + row * d + c);
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += bf16_to_f32(wd[i] & 0xFFFFu);
                acc[2 * i + 1] += bf16_to_f32(wd[i] >> 16);
            }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4 *>(y + (int64_t)t * d + c) = o;
    }
}

template <int BM>
static hipError_t launch_bm(const Plan &p, const uint16_t *x, const moe_weights &w,
                            const moe_routing &r, uint16_t *y, void *ws, hipStream_t s,
                            EventTrace *tr)
{
    char *wsb = static_cast<char *>(ws);
    uint16_t *h_r = reinterpret_cast<uint16_t *>(wsb + p.off_hr);
    uint16_t *h_s = reinterpret_cast<uint16_t *>(wsb + p.off_hs);
    uint16_t *obuf = reinterpret_cast<uint16_t *>(wsb + p.off_obuf);
    const GemmTiles tiles = {r.tile_expert, r.tile_row0, r.tile_rows, r.num_tiles, (int)p.max_tiles};
    const int shared_tiles = (p.T + BM - 1) / BM;

    GateUpArgs g;
    g.x = x; g.perm = r.perm;
    g.T = p.T; g.d = p.d; g.k = p.k; g.G = p.G; g.F = p.F; g.Fs = p.Fs;
    g.gate = w.gate; g.up = w.up; g.sgate = w.sgate; g.sup = w.sup;
    g.tiles = tiles;
    g.ntn_r = (p.F + 127) / 128;
    g.ntn_s = (p.Fs + 127) / 128;
    g.nblk_r = (int)p.max_tiles * g.ntn_r;
    g.nblk_s = shared_tiles * g.ntn_s;
    g.nblk_pad = (g.nblk_r + g.nblk_s + 7) & ~7;
    g.h_r = h_r; g.h_s = h_s;
    launch(tr, moe_gateup_kernel<BM>, dim3(g.nblk_pad), dim3(kGemmThreads), 0, s, g);

    DownArgs dn;
    dn.h_r = h_r; dn.h_s = h_s; dn.perm = r.perm; dn.topk_w = r.topk_w;
    dn.T = p.T; dn.d = p.d; dn.k = p.k; dn.G = p.G; dn.F = p.F; dn.Fs = p.Fs;
    dn.down = w.down; dn.sdown = w.sdown;
    dn.tiles = tiles;
    dn.ntn = (p.d + 255) / 256;
    dn.obuf = obuf;
    dn.nblk_r = (int)p.max_tiles * dn.ntn;
    dn.nblk_s = shared_tiles * dn.ntn;
    dn.nblk_pad = (dn.nblk_r + dn.nblk_s + 7) & ~7;
    launch(tr, moe_down_kernel<BM>, dim3(dn.nblk_pad), dim3(kGemmThreads), 0, s, dn);

    launch(tr, moe_combine_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, (const uint16_t *)obuf,
           (const int32_t *)r.inv_perm, p.T, p.k, p.d, y);
    return hipGetLastError();
}

hipError_t launch_ffn_gemm(const Plan &p, const uint16_t *x, const moe_weights &w,
                           const moe_routing &r, uint16_t *y, void *ws, hipStream_t s,
                           EventTrace *tr)
{
    switch (p.tile_m) {
    case 32: return launch_bm<32>(p, x, w, r, y, ws, s, tr);
    case 64: return launch_bm<64>(p, x, w, r, y, ws, s, tr);
    default: return launch_bm<128>(p, x, w, r, y, ws, s, tr);
    }
}

}  // namespace moe
