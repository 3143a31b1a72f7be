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
// The activations (gathered token rows, read by every wave of the block) and
// the 4-bit codes are copied global->LDS one step (A) and one pair of steps
// (B) ahead, so the copies of the next step overlap the matrix-core work of
// the current one.
//
// Kernels (stream-ordered, no host round trip):
//   moe_gateup_kernel   routed tiles (rows gathered through perm) and shared
//                       tiles (token rows) in one grid:
//                       h = bf16(silu(A W_gate^T) * (A W_up^T))
//   moe_down_kernel     routed and shared tiles in one grid:
//                       o = w_route * (h W_down^T) -> bf16 rows: routed rows
//                       in sorted order, then the T shared rows (weight 1)
//   moe_combine_kernel  y[t] = bf16(sum_j o[inv_perm[t k + j]] + gamma_t o[T k + t]),
//                       slot order then shared, fp32: deterministic, no
//                       atomics; gamma_t = sigmoid(x_t . shared_gate) when
//                       the shared expert is gated, else 1.
//
// MFMA 32x32x16 operand layout used (wave64): lane l holds row (A) or
// column (B) l % 32 and the 8 contraction slots of half h = l / 32; the
// contraction index of slot j in sub-step s of a 64-wide K step is
// k = 32 h + 8 s + j for BOTH operands (any common assignment is valid),
// which makes each lane's B codes one contiguous 16-byte load and its A
// operand one contiguous 16-byte LDS read.  The weights are the first
// operand, so the accumulators hold the transposed tile: register r of lane
// l is D[row l % 32][column 8 (r / 4) + 4 (l / 32) + r % 4], one output row
// per lane, which the epilogues store straight from registers.
#include <type_traits>

#include "gemm_common.h"

namespace moe {

constexpr int kGemmThreads = 256;      // 4 waves
// ---- LDS layout -----------------------------------------------------------
// Every buffer below is its own LDS object, filled by global->LDS copies
// (global_load_lds_dwordx4) and indexed statically, so the compiler can tell
// a buffer being read from the one being filled and does not wait for
// copies that are still in flight.
// A stages (2): [MS*32 rows][64 bf16] (128-byte rows); the eight 16-byte
// chunks of row r are stored XOR-permuted, chunk c at slot c ^ ((r >> 1) & 7),
// which keeps the MFMA operand reads (16 rows x one chunk) free of bank
// conflicts.
// B buffers (2, one per pair of K steps): [4 waves][64 rows][64 bytes] of raw
// 4-bit codes; chunk c of row r at slot c ^ ((r >> 2) & 3).
constexpr int kARow = 128;                        // bytes per A row in LDS
constexpr int kBRow = 64;                         // bytes of codes per B row per pair of K steps
constexpr int kBWave = 64 * kBRow;                // 4 KB per wave
constexpr int kBBuf = 4 * kBWave;                 // 16 KB per buffer

// Copy the A tile of K step kt (MS*32 rows x 64 bf16) into an A stage:
// wave w, copy i moves rows 8 (4 i + w) .. +7, 8 lanes per 128-byte row.
// aoff[i] is this lane's byte offset (source row, chunk) from abase for copy
// i (rows past the tile's end point at a valid row; their products land in
// discarded output rows).
template <int MS>
__device__ __forceinline__ void a_dma(const uint16_t *abase, const uint32_t (&aoff)[MS], int kt, uint8_t *stage)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint16_t *base = abase + kt * kKStep;
#pragma unroll
    for (int i = 0; i < MS; ++i) dma16(base, aoff[i], stage + (4 * i + wave) * 1024);
}

// Per-wave B source: the 64 rows this wave multiplies (rows 0..31 feed the
// first accumulator set, 32..63 the second) and their scale/bias rows, as
// wave-uniform bases plus per-lane byte offsets.
struct BSrc {
    const uint8_t *q[4];   // code row 16 q of this wave (copy q moves rows 16 q .. 16 q + 15)
    uint32_t qrow;         // this lane's row inside a copy (lane / 4) times the row pitch
    uint32_t c16;          // byte offset of the source chunk stored in this lane's slot
    const uint16_t *s0, *b0, *s1, *b1;  // scale/bias rows 0 (first set) and 32 (second set)
    uint32_t soff;         // byte offset of this lane's scale/bias row (lane % 32)
    int kbytes;            // bytes of codes per row (K / 2)
    int ngroups;           // groups per row (K / G)
    // chained column blocks (down GEMM): pair p belongs to column block
    // p >> pshift; the wave's rows of column block c start c * cq code bytes
    // and c * cs scale bytes after those of block 0.  pshift = 30: one block.
    int pshift;
    uint32_t cq, cs;
};

// Copy the codes of pair p (K steps 2p, 2p+1: 64 bytes per row) of this
// wave's 64 rows into its slice of an LDS buffer: 4 copies of 16 rows x 64 B;
// chunk c of row r lands in slot c ^ ((r >> 2) & 3) (src.c16 holds the chunk
// of this lane's slot).  In the half pair at the end of an odd step count the
// window is clamped to the row.
__device__ __forceinline__ uint32_t b_offset(const BSrc &src, int p)
{
    const uint32_t c = (uint32_t)p >> src.pshift, pp = (uint32_t)p & ((1u << src.pshift) - 1u);
    return src.qrow + c * src.cq + min(64u * pp + src.c16, (uint32_t)src.kbytes - 16u);
}

__device__ __forceinline__ void b_dma(const BSrc &src, int p, uint8_t *wave_buf)
{
    const uint32_t off = b_offset(src, p);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(src.q[q], off, wave_buf + q * 1024);
}

template <int G>
__device__ __forceinline__ void sb_load(SBPair<G> &t, const BSrc &src, int p)
{
    constexpr int NG = 128 / G;  // groups per pair
    const uint32_t c = (uint32_t)p >> src.pshift;
    const int g0 = (int)((uint32_t)p & ((1u << src.pshift) - 1u)) * NG;
    const uint32_t off = src.soff + c * src.cs;
    auto at = [&](const uint16_t *base, int g) __attribute__((always_inline)) {
        return reinterpret_cast<const uint8_t *>(base) + off + 2 * g;
    };
    if constexpr (G == 128) {
        t.s0[0] = *reinterpret_cast<const uint16_t *>(at(src.s0, g0));
        t.b0[0] = *reinterpret_cast<const uint16_t *>(at(src.b0, g0));
        t.s1[0] = *reinterpret_cast<const uint16_t *>(at(src.s1, g0));
        t.b1[0] = *reinterpret_cast<const uint16_t *>(at(src.b1, g0));
    } else {
#pragma unroll
        for (int w = 0; w < SBPair<G>::NW; ++w) {
            const int g = g0 + 2 * w;
            if (g + 1 < src.ngroups) {  // both groups of the word exist: one 4-byte load
                t.s0[w] = *reinterpret_cast<const uint32_t *>(at(src.s0, g));
                t.b0[w] = *reinterpret_cast<const uint32_t *>(at(src.b0, g));
                t.s1[w] = *reinterpret_cast<const uint32_t *>(at(src.s1, g));
                t.b1[w] = *reinterpret_cast<const uint32_t *>(at(src.b1, g));
            } else {  // tail of a row with an odd group count
                const int gg = min(g, src.ngroups - 1);
                t.s0[w] = *reinterpret_cast<const uint16_t *>(at(src.s0, gg));
                t.b0[w] = *reinterpret_cast<const uint16_t *>(at(src.b0, gg));
                t.s1[w] = *reinterpret_cast<const uint16_t *>(at(src.s1, gg));
                t.b1[w] = *reinterpret_cast<const uint16_t *>(at(src.b1, gg));
            }
        }
    }
}

// This lane's codes of one K step (16 bytes per half-matrix), read from the
// wave's slice of the LDS buffer of the step's pair.
struct StepCodes {
    uint32_t w0[4], w1[4];
};

// scale and bias of K step j of a pair for this lane's two columns
struct StepScales {
    float s0, b0, s1, b1;
};

template <int G>
__device__ __forceinline__ StepScales step_scales(const SBPair<G> &sb, int j)
{
    const int h = (threadIdx.x & 63) >> 5;
    StepScales t;
    sb_pick<G>(sb.s0, sb.b0, j, h, t.s0, t.b0);
    sb_pick<G>(sb.s1, sb.b1, j, h, t.s1, t.b1);
    return t;
}

__device__ __forceinline__ void read_codes(const uint8_t *bwave, int j, StepCodes &sc)
{
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, n = lane & 31;
    const int c = 2 * j + h;  // code chunk of this step and half
    const uint4 *bq = reinterpret_cast<const uint4 *>(__builtin_assume_aligned(bwave, 16));
    const uint4 q0 = bq[n * (kBRow / 16) + (c ^ ((n >> 2) & 3))];
    const int n1 = 32 + n;
    const uint4 q1 = bq[n1 * (kBRow / 16) + (c ^ ((n1 >> 2) & 3))];
    sc.w0[0] = q0.x; sc.w0[1] = q0.y; sc.w0[2] = q0.z; sc.w0[3] = q0.w;
    sc.w1[0] = q1.x; sc.w1[1] = q1.y; sc.w1[2] = q1.z; sc.w1[3] = q1.w;
}

// The decoded B operands of the first sub-step of a K step.
struct FirstOps {
    bf16x8 o0, o1;
};

__device__ __forceinline__ void decode_first(const StepCodes &sc, const StepScales &t, FirstOps &f)
{
    f.o0 = decode_sub(sc.w0[0], t.s0, t.b0);
    f.o1 = decode_sub(sc.w1[0], t.s1, t.b1);
}

// Copies a K step issues for later steps: the A tile of the next step and,
// at the first step of a pair (B), the codes of the pair two ahead.
template <int MS, bool B>
struct StepCopies {
    const uint16_t *a_src;       // A base at the next step's K offset
    const uint32_t (&aoff)[MS];  // this lane's A offsets
    uint8_t *a_dst;              // next A stage
    const BSrc &b;
    uint32_t b_off;              // this lane's code offset in the pair two ahead
    uint8_t *b_dst;              // that pair's buffer (this wave's slice)

    // The copies of sub-step s: A in sub-steps 0 and 1, codes in 2 and 3, at
    // most two per sub-step.  Issued all at once, the copies of a step (up to
    // 64 KB per CU) queue behind each other and a wave whose copy cannot
    // enter the full queue stalls with all its matrix-core work behind it.
    // The codes stay the last copies of the step, which the entry wait of
    // the next step relies on.
    __device__ __forceinline__ void issue(int s) const
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int i = 0; i < MS; ++i)
            if ((2 * i) / MS == s) dma16(a_src, aoff[i], a_dst + (4 * i + wave) * 1024);
        if constexpr (B) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (2 + q / 2 == s) dma16(b.q[q], b_off, b_dst + q * 1024);
        }
    }
};

// One 64-wide K step.  The codes of this step (cur) were read and its first
// sub-step decoded (first) during the previous step; the four 16-wide MFMA
// sub-steps are software pipelined (decode and A reads of sub-step s+1 under
// the MFMAs of s), and under the MFMAs of the last sub-step the codes of the
// next step are read from LDS (bnext, step jn of its pair) and its first
// sub-step is decoded, so the next step starts with matrix-core work.  The
// copies for later steps are spread over the sub-steps (cp).
template <int MS, int G, bool B, bool WAITB>
__device__ __forceinline__ void kstep(const uint8_t *astage, const StepCodes &cur, const StepScales &sc,
                                      const FirstOps &first, const uint8_t *bnext, SBPair<G> &sbnext, int jn,
                                      StepCodes &nxt, FirstOps &nfirst, f32x16 (&acc0)[MS], f32x16 (&acc1)[MS],
                                      const StepCopies<MS, B> &cp)
{
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, n = lane & 31;
    // A operand of sub-tile i, sub-step s: row 32 i + n, chunk 4 h + s
    const bf16x8 *aq = reinterpret_cast<const bf16x8 *>(__builtin_assume_aligned(astage, 16));
    auto aread = [&](int i, int s) __attribute__((always_inline)) {
        const int row = 32 * i + n;
        return aq[row * (kARow / 16) + ((4 * h + s) ^ ((row >> 1) & 7))];
    };
    bf16x8 o0[2], o1[2];
    o0[0] = first.o0;
    o1[0] = first.o1;
    // A operands one sub-step ahead: each register is reloaded for sub-step
    // s+1 right after the two MFMAs of sub-step s that read it, so the LDS
    // latency hides under the MFMAs of the other sub-tiles and no register
    // is added (only the first sub-step's reads follow the barrier directly)
    bf16x8 av[MS];
#pragma unroll
    for (int i = 0; i < MS; ++i) av[i] = aread(i, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, MS, 0);  // these reads first, all in flight together
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cu = s & 1, nx = cu ^ 1;
        cp.issue(s);
        if (s < 3) {
            o0[nx] = decode_sub(cur.w0[s + 1], sc.s0, sc.b0);
            o1[nx] = decode_sub(cur.w1[s + 1], sc.s1, sc.b1);
        } else {
            // two code buffers: the codes of the next pair were copied during
            // the previous step; the MS A copies of this step may stay in flight
            if constexpr (WAITB) wait_vmcnt<MS>();
            read_codes(bnext, jn, nxt);
            // the next pair's scales are consumed here and not earlier: their
            // loads may still be in flight before this point
#pragma unroll
            for (int w = 0; w < SBPair<G>::NW; ++w)
                asm volatile("" : "+v"(sbnext.s0[w]), "+v"(sbnext.b0[w]), "+v"(sbnext.s1[w]), "+v"(sbnext.b1[w]));
            decode_first(nxt, step_scales<G>(sbnext, jn), nfirst);
        }
#pragma unroll
        for (int i = 0; i < MS; ++i) {
            acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o0[cu], av[i], acc0[i], 0, 0, 0);
            acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o1[cu], av[i], acc1[i], 0, 0, 0);
            if (s < 3) av[i] = aread(i, s + 1);
        }
        if (s < 3) interleave_pairs<MS, 1>(); else interleave_pairs<MS, 0>();
    }
}

// LDS objects of one block: two A stages, three B buffers (this wave's
// slices).  Separate objects, each indexed statically, so that reading one
// never waits for copies still landing in another.
struct LdsBufs {
    uint8_t *a0, *a1, *b0, *b1, *b2;
    template <int I> __device__ __forceinline__ uint8_t *a() const { return I == 0 ? a0 : a1; }
    template <int I> __device__ __forceinline__ uint8_t *b() const { return I == 0 ? b0 : I == 1 ? b1 : b2; }
};

// Pipeline state carried from one K step to the next.
template <int G>
struct Carry {
    SBPair<G> sb, sbn;  // scales of the current pair and of the next one
    StepCodes codes;    // codes of the next step
    FirstOps first;     // its decoded first sub-step
};

// One K step.  ST = kt % 6 fixes J = kt & 1 (A stage, step inside the pair)
// and PB = (kt / 2) % 3 (B buffer of the pair).  Codes are copied two pairs
// ahead, A one step ahead, scales one pair ahead (registers).  Issue order
// at J = 0: the scale loads of pair p+1, then (spread over the sub-steps) the
// copies of A(kt+1) and those of pair p+2 (into the buffer of pair p-1, last
// read one step before this one); at J = 1 the copies of A(kt+1).  Entry
// wait: at J = 1 the scales and this wave's copy of A(kt) must have landed,
// the 4 code copies issued after them need not; at J = 0 everything, which
// includes the codes of pair p+1 that the end of the next step reads.  After
// the barrier every wave's copies up to there are in LDS.
// Steps of one main loop: nt K steps in npair pairs.  With chained column
// blocks (nc > 1, steps per block nk a power of two) step kt multiplies the
// A columns of K step kt & kmask into the weights of column block kt / nk.
struct LoopShape {
    int nt, npair, kmask, kshift;
};

// A chained loop's end of a column block: the epilogue stores the block's
// accumulators (column block c), then they are cleared for the next one.
struct NoEpilogue {
    template <int MS>
    __device__ __forceinline__ void operator()(int, f32x16 (&)[MS], f32x16 (&)[MS]) const {}
};

// One K step.  ST = kt % 6 fixes J = kt & 1 (A stage, step inside the pair)
// and PB = (kt / 2) % 3 (B buffer of the pair).  Codes are copied two pairs
// ahead, A one step ahead, scales one pair ahead (registers).  Issue order
// at J = 0: the scale loads of pair p+1, then (spread over the sub-steps) the
// copies of A(kt+1) and those of pair p+2 (into the buffer of pair p-1, last
// read one step before this one); at J = 1 the copies of A(kt+1).  Entry
// wait: at J = 1 the scales and this wave's copy of A(kt) must have landed,
// the 4 code copies issued after them need not; at J = 0 everything, which
// includes the codes of pair p+1 that the end of the next step reads.  After
// the barrier every wave's copies up to there are in LDS.  A chained loop
// stores a finished column block at the end of its last step (kt + 1 a
// multiple of nk, always a J = 1 step); its stores are in the vector-memory
// count, so the entry wait of the next step (J = 0: everything) also covers
// them.
template <int MS, int G, int NB, int ST, class Epi>
__device__ __forceinline__ void mainloop_step(int kt, const LoopShape &ls, const uint16_t *abase,
                                              const uint32_t (&aoff)[MS], const BSrc &bsrc, const LdsBufs &L,
                                              Carry<G> &cs, f32x16 (&acc0)[MS], f32x16 (&acc1)[MS], const Epi &epi)
{
    constexpr int J = ST & 1, PB = (ST >> 1) % NB;
    if constexpr (J == 1) wait_vmcnt<4>(); else wait_vmcnt<0>();
    block_sync();
    if constexpr (J == 0) sb_load<G>(cs.sbn, bsrc, min((kt >> 1) + 1, ls.npair - 1));
    const StepCopies<MS, J == 0> cp = {abase + (min(kt + 1, ls.nt - 1) & ls.kmask) * kKStep, aoff, L.a<J ^ 1>(),
                                       bsrc, b_offset(bsrc, min((kt >> 1) + NB - 1, ls.npair - 1)),
                                       L.b<(PB + NB - 1) % NB>()};
    // next step: same pair at J = 0, first step of the next pair at J = 1
    constexpr int PBN = J == 0 ? PB : (PB + 1) % NB;
    const StepCodes cur = cs.codes;
    const FirstOps first = cs.first;
    const StepScales sc = step_scales<G>(cs.sb, J);
    kstep<MS, G, J == 0, NB == 2 && J == 1>(L.a<J>(), cur, sc, first, L.b<PBN>(), J == 0 ? cs.sb : cs.sbn, J ^ 1, cs.codes, cs.first,
                         acc0, acc1, cp);
    if constexpr (J == 1) cs.sb = cs.sbn;
    if constexpr (J == 1 && !std::is_same<Epi, NoEpilogue>::value) {
        if (((kt + 1) & ls.kmask) == 0) {
            epi(kt >> ls.kshift, acc0, acc1);
#pragma unroll
            for (int i = 0; i < MS; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) { acc0[i][r] = 0.f; acc1[i][r] = 0.f; }
        }
    }
}

// Main loop shared by both GEMMs: acc0 += A B0^T, acc1 += A B1^T over K for
// MS live 32-row sub-tiles.  The (A stage, B buffer) assignment repeats every
// 6 steps: the loop body is 6 straight-line steps, and 1 to 5 remaining
// steps run the same instantiations under conditions.  Past the end, copies
// re-load valid data instead of branching.
template <int MS, int G, int NB, class Epi = NoEpilogue>
__device__ __forceinline__ void mainloop(const uint16_t *abase, const uint32_t (&aoff)[MS], const LoopShape &ls,
                                         const BSrc &bsrc, const LdsBufs &L, f32x16 (&acc0)[MS],
                                         f32x16 (&acc1)[MS], const Epi &epi = Epi())
{
    const int nk = ls.nt;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { acc0[i][r] = 0.f; acc1[i][r] = 0.f; }

    Carry<G> cs;
    sb_load<G>(cs.sb, bsrc, 0);
    a_dma<MS>(abase, aoff, 0, L.a<0>());
    b_dma(bsrc, 0, L.b<0>());
    if constexpr (NB == 3) b_dma(bsrc, min(1, ls.npair - 1), L.b<1>());
    wait_vmcnt<0>();
    block_sync();
    read_codes(L.b<0>(), 0, cs.codes);
    decode_first(cs.codes, step_scales<G>(cs.sb, 0), cs.first);

    int kt = 0;
    if constexpr (NB == 3) {
        for (; kt + 5 < nk; kt += 6) {
            mainloop_step<MS, G, NB, 0>(kt, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 1>(kt + 1, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 2>(kt + 2, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 3>(kt + 3, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 4>(kt + 4, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 5>(kt + 5, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        }
        if (kt < nk) mainloop_step<MS, G, NB, 0>(kt, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 1 < nk) mainloop_step<MS, G, NB, 1>(kt + 1, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 2 < nk) mainloop_step<MS, G, NB, 2>(kt + 2, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 3 < nk) mainloop_step<MS, G, NB, 3>(kt + 3, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 4 < nk) mainloop_step<MS, G, NB, 4>(kt + 4, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
    } else {
        for (; kt + 3 < nk; kt += 4) {
            mainloop_step<MS, G, NB, 0>(kt, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 1>(kt + 1, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 2>(kt + 2, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
            mainloop_step<MS, G, NB, 3>(kt + 3, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        }
        if (kt < nk) mainloop_step<MS, G, NB, 0>(kt, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 1 < nk) mainloop_step<MS, G, NB, 1>(kt + 1, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
        if (kt + 2 < nk) mainloop_step<MS, G, NB, 2>(kt + 2, ls, abase, aoff, bsrc, L, cs, acc0, acc1, epi);
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the loop
}

// the shape of a loop over one column block of K (no chaining)
__device__ __forceinline__ LoopShape single_block_loop(int K)
{
    const int nk = K / kKStep;
    return {nk, (nk + 1) >> 1, 0x7fffffff, 30};
}

// Byte offsets from the A base of this lane's source (row, chunk) for the A
// copies of sub-tiles < MS: copy i fills rows 8 (4 i + w) + lane / 8 of the
// stage, 8 lanes per 128-byte row, and the lane in slot c of its row copies
// chunk c ^ ((row >> 1) & 7).  Rows are gathered through perm (routed tiles)
// (values clamped to the nassign assignments) or contiguous; rows past the
// tile's end repeat its last row.
template <int MS>
__device__ __forceinline__ void a_offsets(uint32_t (&aoff)[MS], int ld, const int32_t *perm, int k, int nassign,
                                          int row0, int rows)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < MS; ++i) {
        const int row = 8 * (4 * i + wave) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        const int m = min(row, rows - 1);
        const int src = perm ? perm_at(perm, row0 + m, nassign) / k : row0 + m;
        aoff[i] = (uint32_t)src * (uint32_t)ld * 2u + (uint32_t)c * 16u;
    }
}

template <int MS, int G, int NB>
__device__ __forceinline__ void gateup_body(const GateUpArgs &a, int row0, int rows, int N,
                                            const moe_qmat &mg, const moe_qmat &mu, size_t ebase,
                                            uint16_t *out, bool routed, int nt, uint8_t *lds_a0,
                                            uint8_t *lds_a1, uint8_t *lds_b0, uint8_t *lds_b1, uint8_t *lds_b2)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wslice = wave * kBWave;
    const LdsBufs L = {lds_a0, lds_a1, lds_b0 + wslice, lds_b1 + wslice, lds_b2 + wslice};
    uint32_t aoff[MS];
    a_offsets<MS>(aoff, a.d, routed ? a.perm : nullptr, a.k, a.T * a.k, row0, rows);
    const int ncol0 = nt * 128 + 32 * wave;  // first h column of this wave
    const int nbase = ncol0 < N ? ncol0 : 0;  // idle waves compute on valid rows
    const int Kq = a.d >> 1, Kg = a.d / G;
    BSrc src;
#pragma unroll
    for (int q = 0; q < 4; ++q)  // copy q moves rows 16 q ..: q < 2 gate, q >= 2 up
        src.q[q] = (q < 2 ? mg : mu).q + uniform_size((ebase + nbase + 16 * (q & 1)) * Kq);
    src.qrow = (uint32_t)(lane >> 2) * Kq;
    src.c16 = 16u * ((lane & 3) ^ ((lane >> 4) & 3));
    const size_t boff = uniform_size((ebase + nbase) * Kg);
    src.s0 = mg.s + boff; src.b0 = mg.b + boff;
    src.s1 = mu.s + boff; src.b1 = mu.b + boff;
    src.soff = (uint32_t)(lane & 31) * Kg * 2u;
    src.kbytes = Kq;
    src.ngroups = Kg;
    src.pshift = 30; src.cq = 0; src.cs = 0;
    f32x16 accg[MS], accu[MS];
    mainloop<MS, G, NB>(a.x, aoff, single_block_loop(a.d), src, L, accg, accu);
    // epilogue: h = bf16(silu(g) * u), one row per lane, 16-byte stores
    if (ncol0 < N) {
#pragma unroll
        for (int i = 0; i < MS; ++i) {
            const int m = 32 * i + (lane & 31);
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = silu(accg[i][r]) * accu[i][r];
            if (m < rows) store_row32(out + (size_t)(row0 + m) * N + ncol0, v);
        }
    }
}

// Code buffers and blocks per CU by GEMM and tile height.  A 32-row down
// block is short (F / 64 K steps per column block) and does one MFMA per
// decoded operand, so its prologue and copy latency have little to hide
// behind: it keeps two code buffers (codes one pair ahead, 40 KB of LDS)
// so that four blocks share a CU.  Measured on the T = 512 workload (32-row
// tiles): down GEMM 57 -> 52 us; the gate/up GEMM (32 K steps) ran slower
// that way (116 -> 156 us) and keeps three buffers and two blocks per CU.
template <int BM, bool DOWN> constexpr int code_buffers() { return BM == 32 && DOWN ? 2 : 3; }
template <int BM, bool DOWN> constexpr int blocks_per_cu() { return BM == 32 && DOWN ? 4 : 2; }

template <int BM, int G>
__global__ __launch_bounds__(kGemmThreads, (blocks_per_cu<BM, false>())) void moe_gateup_kernel(GateUpArgs a)
{
    constexpr int kNB = code_buffers<BM, false>();
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * kARow];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[BM * kARow];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[kBBuf];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[kBBuf];
    uint8_t *lds_b2 = lds_b1;  // unused with two code buffers
    if constexpr (kNB == 3) {
        __shared__ __attribute__((aligned(1024))) uint8_t lds_b2x[kBBuf];
        lds_b2 = lds_b2x;
    }
    const int nblk_r = max(0, min(*a.tiles.num_tiles, a.tiles.max_tiles)) * a.ntn_r;  // routed blocks with work
    const int L = xcd_logical_block(blockIdx.x, nblk_r + a.nblk_s);
    if (L < 0) return;
    int row0, rows, N, nt;
    const moe_qmat *mg, *mu;
    size_t ebase;  // first row of the expert's slab
    uint16_t *out;
    bool routed;
    if (L < nblk_r) {
        const int tile = L / a.ntn_r;
        nt = L - tile * a.ntn_r;
        const TileInfo ti = read_tile(a.tiles, tile, a.E, a.T * a.k, BM);
        row0 = ti.row0;
        rows = ti.rows;
        N = a.F; mg = &a.gate; mu = &a.up;
        ebase = (size_t)ti.e * a.F;
        out = a.h_r;
        routed = true;
    } else {
        const int tile = (L - nblk_r) / a.ntn_s;
        nt = (L - nblk_r) - tile * a.ntn_s;
        row0 = tile * BM;
        rows = min(BM, a.T - row0);
        N = a.Fs; mg = &a.sgate; mu = &a.sup;
        ebase = 0;
        out = a.h_s;
        routed = false;
    }
    const int msub = (rows + 31) >> 5;  // live 32-row sub-tiles (block-uniform)
    if (BM >= 128 && msub > 2)
        gateup_body<(BM >= 128 ? 4 : 1), G, kNB>(a, row0, rows, N, *mg, *mu, ebase, out, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
    else if (BM >= 64 && msub == 2)
        gateup_body<(BM >= 64 ? 2 : 1), G, kNB>(a, row0, rows, N, *mg, *mu, ebase, out, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
    else
        gateup_body<1, G, kNB>(a, row0, rows, N, *mg, *mu, ebase, out, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
}

// Store 64 columns (this wave's share of a 256-column block) of the tile's
// rows: o = w_route * acc as bf16, one row per lane, 16-byte stores.
template <int MS>
__device__ __forceinline__ void down_store(const DownArgs &a, const float (&wrow)[MS], int rows, int orow0,
                                           int ncol0, const f32x16 (&acc0)[MS], const f32x16 (&acc1)[MS])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
        const int m = 32 * i + (lane & 31);
        if (m >= rows) continue;
        uint16_t *orow = a.obuf + (size_t)(orow0 + m) * a.d + ncol0;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = wrow[i] * acc0[i][r];
        store_row32(orow, v);
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = wrow[i] * acc1[i][r];
        store_row32(orow + 32, v);
    }
}

// Down GEMM over one tile and NC = a.nc consecutive 256-column blocks
// starting at block nt0.  CHAIN (NC > 1): one continuous pipeline over
// NC x (K / 64) steps -- the h tile is the A operand of every column block,
// the codes and scales move to the next block's rows, and each finished
// block is stored from inside the loop, so the block's prologue (tile
// lookup, routing weights, first copies) is paid once per NC blocks.
template <int MS, int G, bool CHAIN, int NB>
__device__ __forceinline__ void down_body(const DownArgs &a, int row0, int rows, int K,
                                          const moe_qmat &m, size_t ebase, const uint16_t *hsrc,
                                          int orow0, bool routed, int nt0, uint8_t *lds_a0,
                                          uint8_t *lds_a1, uint8_t *lds_b0, uint8_t *lds_b1, uint8_t *lds_b2)
{
    const int lane = threadIdx.x & 63;
    // routing weight of this lane's output row in each sub-tile (the shared
    // expert's rows have weight 1), loaded before the main loop
    float wrow[MS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
        wrow[i] = routed ? a.topk_w[perm_at(a.perm, row0 + min(32 * i + (lane & 31), rows - 1), a.T * a.k)] : 1.0f;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wslice = wave * kBWave;
    const LdsBufs L = {lds_a0, lds_a1, lds_b0 + wslice, lds_b1 + wslice, lds_b2 + wslice};
    uint32_t aoff[MS];
    a_offsets<MS>(aoff, K, nullptr, 1, 0, row0, rows);
    const int ncol0 = nt0 * 256 + 64 * wave;  // this wave: columns [ncol0, ncol0 + 64) of the first block
    const int nbase = ncol0 < a.d ? ncol0 : 0;  // idle waves compute on valid rows
    const int Kq = K >> 1, Kg = K / G;
    BSrc src;
#pragma unroll
    for (int q = 0; q < 4; ++q) src.q[q] = m.q + uniform_size((ebase + nbase + 16 * q) * Kq);
    src.qrow = (uint32_t)(lane >> 2) * Kq;
    src.c16 = 16u * ((lane & 3) ^ ((lane >> 4) & 3));
    const size_t o0 = uniform_size((ebase + nbase) * Kg), o1 = o0 + 32 * Kg;
    src.s0 = m.s + o0; src.b0 = m.b + o0;
    src.s1 = m.s + o1; src.b1 = m.b + o1;
    src.soff = (uint32_t)(lane & 31) * Kg * 2u;
    src.kbytes = Kq;
    src.ngroups = Kg;
    f32x16 acc0[MS], acc1[MS];
    if constexpr (CHAIN) {
        // steps per column block: a power of two (host-checked), so pairs
        // never straddle two blocks
        const int nk = K / kKStep;
        const int kshift = 31 - __builtin_clz(nk);
        src.pshift = kshift - 1;
        src.cq = 256u * (uint32_t)Kq;
        src.cs = 256u * (uint32_t)Kg * 2u;
        const LoopShape ls = {nk * a.nc, nk * a.nc / 2, nk - 1, kshift};
        auto epi = [&](int c, auto &r0, auto &r1) __attribute__((always_inline)) {
            down_store<MS>(a, wrow, rows, orow0, ncol0 + 256 * c, r0, r1);
        };
        mainloop<MS, G, NB>(hsrc, aoff, ls, src, L, acc0, acc1, epi);
    } else {
        src.pshift = 30; src.cq = 0; src.cs = 0;
        mainloop<MS, G, NB>(hsrc, aoff, single_block_loop(K), src, L, acc0, acc1);
        if (ncol0 < a.d) down_store<MS>(a, wrow, rows, orow0, ncol0, acc0, acc1);
    }
}

template <int BM, int G>
__global__ __launch_bounds__(kGemmThreads, (blocks_per_cu<BM, true>())) void moe_down_kernel(DownArgs a)
{
    constexpr int kNB = code_buffers<BM, true>();
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * kARow];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[BM * kARow];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[kBBuf];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[kBBuf];
    uint8_t *lds_b2 = lds_b1;  // unused with two code buffers
    if constexpr (kNB == 3) {
        __shared__ __attribute__((aligned(1024))) uint8_t lds_b2x[kBBuf];
        lds_b2 = lds_b2x;
    }
    const int ncb = a.ntn / a.nc;  // blocks per tile, each over a.nc column blocks
    const int nblk_r = max(0, min(*a.tiles.num_tiles, a.tiles.max_tiles)) * ncb;  // routed blocks with work
    const int L = xcd_logical_block(blockIdx.x, nblk_r + a.nblk_s);
    if (L < 0) return;
    int row0, rows, K, nt;
    const moe_qmat *m;
    size_t ebase;
    const uint16_t *hsrc;
    int orow0;  // first output row in obuf
    bool routed;
    if (L < nblk_r) {
        const int tile = L / ncb;
        nt = (L - tile * ncb) * a.nc;
        const TileInfo ti = read_tile(a.tiles, tile, a.E, a.T * a.k, BM);
        ebase = (size_t)ti.e * a.d;
        row0 = ti.row0;
        rows = ti.rows;
        K = a.F; m = &a.down; hsrc = a.h_r;
        orow0 = row0;
        routed = true;
    } else {
        const int tile = (L - nblk_r) / ncb;
        nt = ((L - nblk_r) - tile * ncb) * a.nc;
        row0 = tile * BM;
        rows = min(BM, a.T - row0);
        ebase = 0;
        K = a.Fs; m = &a.sdown; hsrc = a.h_s;
        orow0 = a.T * a.k + row0;
        routed = false;
    }
    const int msub = (rows + 31) >> 5;
    if (a.nc > 1) {
        if (BM >= 128 && msub > 2)
            down_body<(BM >= 128 ? 4 : 1), G, true, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
        else if (BM >= 64 && msub == 2)
            down_body<(BM >= 64 ? 2 : 1), G, true, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
        else
            down_body<1, G, true, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
    } else {
        if (BM >= 128 && msub > 2)
            down_body<(BM >= 128 ? 4 : 1), G, false, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
        else if (BM >= 64 && msub == 2)
            down_body<(BM >= 64 ? 2 : 1), G, false, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
        else
            down_body<1, G, false, kNB>(a, row0, rows, K, *m, ebase, hsrc, orow0, routed, nt, lds_a0, lds_a1, lds_b0, lds_b1, lds_b2);
    }
}

// One wave per token: 16-byte loads of the k routed rows and the shared row.
// The row indices are read once, with every lane active (lane j of register
// g holds inv_perm[t k + 64 g + j]), and taken out lane by lane with
// v_readlane on those registers, so the row loads of a pass do not wait on
// index loads.  The column passes are wave-uniform (loads and stores are
// predicated on c < d) and each index is clamped to the routed rows, so a
// corrupt routing input cannot send a load outside obuf.  Each lane sums 8
// columns per pass in slot order (fp32), then the shared row.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ obuf,
                                                          const int32_t *__restrict__ inv_perm,
                                                          int T, int k, int d,
                                                          const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ shared_gate,
                                                          uint16_t *__restrict__ y)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;  // wave-uniform
    const int64_t shared_row = (int64_t)T * k + t;
    const uint32_t last_routed = (uint32_t)(T * k - 1);
    int myrow[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int j = 64 * g + lane;
        myrow[g] = j < k ? inv_perm[(int64_t)t * k + j] : 0;
    }
    float gamma = 1.0f;  // weight of the shared expert's row
    if (shared_gate) {
        float z = 0.f;
        for (int c = lane * 8; c < d; c += 64 * 8) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(x + (int64_t)t * d + c);
            const uint4 gv = *reinterpret_cast<const uint4 *>(shared_gate + c);
            z = dot2_bf16(xv.x, gv.x, z);
            z = dot2_bf16(xv.y, gv.y, z);
            z = dot2_bf16(xv.z, gv.z, z);
            z = dot2_bf16(xv.w, gv.w, z);
        }
        gamma = 1.0f / (1.0f + __expf(-wave_sum(z)));
    }
    for (int c0 = 0; c0 < d; c0 += 64 * 8) {  // wave-uniform passes
        const int c = c0 + lane * 8;
        const bool act = c < d;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        auto add = [&](const uint4 &v, float wr) __attribute__((always_inline)) {
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += wr * bf16_to_f32(wd[i] & 0xFFFFu);
                acc[2 * i + 1] += wr * bf16_to_f32(wd[i] >> 16);
            }
        };
        // slots in groups of 8: the 8 loads of a group are issued together
        for (int j0 = 0; j0 < k; j0 += 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;  // wave-uniform
                const int l = j & 63, g = (j >> 6) & 3;
                const int r0 = __builtin_amdgcn_readlane(myrow[0], l);
                const int r1 = __builtin_amdgcn_readlane(myrow[1], l);
                const int r2 = __builtin_amdgcn_readlane(myrow[2], l);
                const int r3 = __builtin_amdgcn_readlane(myrow[3], l);
                const uint32_t row = min((uint32_t)(g == 0 ? r0 : g == 1 ? r1 : g == 2 ? r2 : r3), last_routed);
                if (j < k && act) v[u] = *reinterpret_cast<const uint4 *>(obuf + (int64_t)row * d + c);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j0 + u < k && act) add(v[u], 1.0f);
        }
        if (act) {
            add(*reinterpret_cast<const uint4 *>(obuf + shared_row * d + c), gamma);
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            *reinterpret_cast<uint4 *>(y + (int64_t)t * d + c) = o;
        }
    }
}

// Column blocks per down-GEMM block (chaining, see down_body): only where
// every wave has columns in every block (d a multiple of 256) and the steps
// of a block (F / 64 = Fs / 64) are a power of two.  Two per block where the
// grid still holds two rounds of blocks (2 per CU) at the largest tile
// count: measured on the T = 4096 and T = 32768 workloads, 4 and 8 were no
// faster than 2 (-3% and -8% down-GEMM time against 1).  moe_dims.down_nc
// (validated on the host) overrides the choice.
static int down_chain(const Plan &p, int BM, int ntn)
{
    const int nk = p.F / kKStep;
    if (p.d % 256 != 0 || p.F != p.Fs || nk < 2 || (nk & (nk - 1)) != 0) return 1;
    if (p.down_nc >= 1 && ntn % p.down_nc == 0) return p.down_nc;
    // chains of 4 where the grid still holds four rounds of blocks (T = 32768:
    // down 772 -> 751 us), of 2 where it holds two (T = 4096), else none (T = 512)
    const int64_t tiles = (p.A + BM - 1) / BM + (p.T + BM - 1) / BM;
    if (ntn % 4 == 0 && tiles * (ntn / 4) >= 4 * 512) return 4;
    return (ntn % 2 == 0 && tiles * (ntn / 2) >= 2 * 512) ? 2 : 1;
}

template <int BM, int G>
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
    g.T = p.T; g.d = p.d; g.E = p.E; g.k = p.k; g.G = p.G; g.F = p.F; g.Fs = p.Fs;
    g.gate = w.gate; g.up = w.up; g.sgate = w.sgate; g.sup = w.sup;
    g.tiles = tiles;
    g.ntn_r = (p.F + 127) / 128;
    g.ntn_s = (p.Fs + 127) / 128;
    g.nblk_s = shared_tiles * g.ntn_s;
    g.nblk_pad = ((int)p.max_tiles * g.ntn_r + g.nblk_s + 7) & ~7;
    g.h_r = h_r; g.h_s = h_s;
    launch(tr, moe_gateup_kernel<BM, G>, dim3(g.nblk_pad), dim3(kGemmThreads), 0, s, g);

    DownArgs dn;
    dn.h_r = h_r; dn.h_s = h_s; dn.perm = r.perm; dn.topk_w = r.topk_w;
    dn.T = p.T; dn.d = p.d; dn.E = p.E; dn.k = p.k; dn.G = p.G; dn.F = p.F; dn.Fs = p.Fs;
    dn.down = w.down; dn.sdown = w.sdown;
    dn.tiles = tiles;
    dn.ntn = (p.d + 255) / 256;
    dn.nc = down_chain(p, BM, dn.ntn);
    dn.obuf = obuf;
    dn.nblk_s = shared_tiles * (dn.ntn / dn.nc);
    dn.nblk_pad = ((int)p.max_tiles * (dn.ntn / dn.nc) + dn.nblk_s + 7) & ~7;
    launch(tr, moe_down_kernel<BM, G>, dim3(dn.nblk_pad), dim3(kGemmThreads), 0, s, dn);

    launch(tr, moe_combine_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, (const uint16_t *)obuf,
           (const int32_t *)r.inv_perm, p.T, p.k, p.d, x, w.shared_gate, y);
    return hipGetLastError();
}

template <int BM>
static hipError_t launch_g(const Plan &p, const uint16_t *x, const moe_weights &w,
                           const moe_routing &r, uint16_t *y, void *ws, hipStream_t s,
                           EventTrace *tr)
{
    switch (p.G) {
    case 32: return launch_bm<BM, 32>(p, x, w, r, y, ws, s, tr);
    case 64: return launch_bm<BM, 64>(p, x, w, r, y, ws, s, tr);
    default: return launch_bm<BM, 128>(p, x, w, r, y, ws, s, tr);
    }
}

hipError_t launch_ffn_gemm(const Plan &p, const uint16_t *x, const moe_weights &w,
                           const moe_routing &r, uint16_t *y, void *ws, hipStream_t s,
                           EventTrace *tr)
{
    switch (p.tile_m) {
    case 32: return launch_g<32>(p, x, w, r, y, ws, s, tr);
    case 64: return launch_g<64>(p, x, w, r, y, ws, s, tr);
    default: return launch_g<128>(p, x, w, r, y, ws, s, tr);
    }
}

}  // namespace moe
