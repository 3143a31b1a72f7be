// Pieces shared by the matrix-core kernels of the prefill path (grouped GEMMs
// and router projection, gfx950):
// kernel arguments, XCD-aware block order, explicit memory-counter waits, the
// fence-free workgroup barrier, scale/bias words of a pair of K steps and the
// register decode of eight 4-bit codes into a bf16 MFMA operand.
#pragma once
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kKStep = 64;             // contraction per main-loop step

struct GemmTiles {
    const int32_t *tile_expert, *tile_row0, *tile_rows, *num_tiles;
    int max_tiles;
};

struct GateUpArgs {
    const uint16_t *x;      // [T][d]
    const int32_t *perm;    // [T*k]
    int T, d, E, k, G, F, Fs;
    moe_qmat gate, up, sgate, sup;
    GemmTiles tiles;
    int ntn_r, ntn_s;       // 128-column blocks per tile (routed, shared)
    int nblk_s;             // blocks of the shared part (the routed part: num_tiles * ntn_r)
    int nblk_pad;           // grid size: routed blocks of max_tiles tiles + nblk_s, multiple of 8
    uint16_t *h_r;          // [T*k][F] sorted rows
    uint16_t *h_s;          // [T][Fs]
};

struct DownArgs {
    const uint16_t *h_r, *h_s;
    const int32_t *perm;
    const float *topk_w;
    int T, d, E, k, G, F, Fs;
    moe_qmat down, sdown;
    GemmTiles tiles;
    int ntn;                // 256-column blocks (d / 256, rounded up)
    int nc;                 // column blocks per block (chained), divides ntn
    int nblk_s, nblk_pad;   // as in GateUpArgs
    uint16_t *obuf;         // [T*k + T][d] weighted outputs: sorted routed rows, then shared
};

// One routed tile of the block map, read from the caller's routing arrays
// and clamped into range: expert < E, first row < A = T k, 1 <= rows <=
// min(tile height, A - first row).  moe_route writes values in range; the
// clamps keep a corrupt routing input from sending a load outside the
// caller's arrays.
struct TileInfo {
    int e, row0, rows;
};

__device__ __forceinline__ TileInfo read_tile(const GemmTiles &t, int tile, int E, int A, int BM)
{
    TileInfo ti;
    ti.e = (int)min((uint32_t)t.tile_expert[tile], (uint32_t)(E - 1));
    ti.row0 = (int)min((uint32_t)t.tile_row0[tile], (uint32_t)(A - 1));
    ti.rows = max(1, min(t.tile_rows[tile], min(BM, A - ti.row0)));
    return ti;
}

// a sorted row's assignment index from perm, clamped to [0, A)
__device__ __forceinline__ int perm_at(const int32_t *perm, int p, int A)
{
    return (int)min((uint32_t)perm[p], (uint32_t)(A - 1));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// A 64-bit integer that is the same in every lane, moved to SGPRs.  The
// builtin returns a signed int: each half is taken back as uint32_t before
// widening, so that bit 31 of the low half never spreads into the high half.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// an offset that is the same in every lane, moved to SGPRs (applied to
// offsets rather than pointers, which keeps the pointers' address space)
__device__ __forceinline__ size_t uniform_size(size_t v) { return (size_t)uniform_u64((uint64_t)v); }

// One 16-byte-per-lane global->LDS copy (global_load_lds_dwordx4, LDS base in
// M0) from base + voff: a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset, so a row address costs one VGPR instead of two.
// Issued from inline assembly so that the compiler does not treat LDS reads
// of the other buffers as dependent on it (it would wait for every copy in
// flight before each of them); the main loop counts these copies itself
// (wait_vmcnt).  No memory clobber: a copy writes an LDS buffer that no wave
// reads until after the next block_sync, whose compiler fences keep every
// LDS access on its side of the barrier, so the LDS reads of the current
// step may be scheduled freely around the copies.  The s_nop covers both the
// M0 write and a base just moved into SGPRs by a VALU readfirstlane.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint8_t *lds)
{
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds);
    const uint64_t sb = uniform_u64((uint64_t)(uintptr_t)base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sb)
                 : "m0");
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier without a memory fence: a fence would also wait for the
// global->LDS copies of later steps; every wave waits for its own copies of
// the current step (wait_vmcnt) before arriving, so after the barrier the
// whole step is in LDS.
__device__ __forceinline__ void block_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");       // no LDS access moves across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// scale/bias words of one pair for the lane's two rows (NW words of two
// bf16 each; group order = pair's groups in ascending order)
template <int G>
struct SBPair {
    static constexpr int NW = G == 32 ? 2 : 1;
    uint32_t s0[NW], b0[NW], s1[NW], b1[NW];
};

// scale (low 16 bits of the result) and bias of K step j of the pair, half h
template <int G>
__device__ __forceinline__ void sb_pick(const uint32_t (&s)[SBPair<G>::NW], const uint32_t (&b)[SBPair<G>::NW],
                                        int j, int h, float &sf, float &bf)
{
    const int gi = (64 * j + 32 * h) / G;  // group index inside the pair
    const uint32_t sw = s[gi >> 1 < SBPair<G>::NW ? gi >> 1 : 0];
    const uint32_t bw = b[gi >> 1 < SBPair<G>::NW ? gi >> 1 : 0];
    const int sh = (gi & 1) * 16;
    sf = __uint_as_float((sw >> sh) << 16);
    bf = __uint_as_float((bw >> sh) << 16);
}

__device__ __forceinline__ bf16x8 decode_sub(uint32_t w, float s, float b)
{
    uint32_t o[4];
    dequant8_bf16(w, s, b, o);
    return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// Store 32 columns of one output row from an accumulator of the transposed
// product (weights as the first MFMA operand): lane l holds row l % 32 of its
// sub-tile, and registers 4 g .. 4 g + 3 hold columns 8 g + 4 h .. 8 g + 4 h
// + 3, h = l / 32.  The values are packed to bf16, then the two halves of
// the wave swap chunks (v_permlane32_swap: the upper half of the first
// operand with the lower half of the second) so that each lane holds 16
// contiguous bytes, columns 16 p + 8 h .. 16 p + 8 h + 7 for p = 0, 1.
// rowp: column 0 of the lane's row (16-byte aligned).
__device__ __forceinline__ void store_row32(uint16_t *rowp, const float (&v)[16])
{
    const int h = (threadIdx.x & 63) >> 5;
    uint32_t d[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        d[g][0] = pack_bf16x2(v[4 * g], v[4 * g + 1]);
        d[g][1] = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto r = __builtin_amdgcn_permlane32_swap(d[2 * p][w], d[2 * p + 1][w], false, false);
            d[2 * p][w] = r[0];
            d[2 * p + 1][w] = r[1];
        }
#pragma unroll
    for (int p = 0; p < 2; ++p)
        *reinterpret_cast<uint4 *>(rowp + 16 * p + 8 * h) = make_uint4(d[2 * p][0], d[2 * p][1], d[2 * p + 1][0], d[2 * p + 1][1]);
}

// scheduling hint for a sub-step of MS pairs of MFMAs: each pair (the two
// MFMAs that read one A operand) is followed by NDS LDS reads (the operand's
// reload for the next sub-step) and 12 VALU ops (decode of the next sub-step)
template <int MS, int NDS>
__device__ __forceinline__ void interleave_pairs()
{
#pragma unroll
    for (int i = 0; i < MS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
        if (NDS) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // 12 VALU
    }
}

}  // namespace moe
