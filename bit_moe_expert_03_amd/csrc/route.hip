// GPU-resident expert routing for the MoE layer (gfx950).
//
// The Lily pages keep the whole routing on the GPU -- histogram, prefix scan,
// scatter and block-map build in one submission, with no host round trip
// (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
// Silicon", section "Prefill optimizations", second bullet).  Here that is
// three stream-ordered kernels and no host synchronisation:
//
//   1. route_topk_kernel    one wave per token: the k best of E logits
//                           (ties -> lower id; DPP wave maxima), softmax
//                           over them, and a per-block expert histogram in
//                           LDS;
//   2. route_scan_kernel    one block: expert totals, the exclusive scan
//                           over experts, the per-block bases of the stable
//                           scatter (column scan over blocks) and the tile
//                           block map;
//   3. route_scatter_kernel one block per route chunk: ranks inside the
//                           chunk from wave ballots (a multisplit), then
//                           perm / inv_perm.
//
// Every step is integer-exact and deterministic (LDS integer atomics only
// count, they never order).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// hist layout: [E][NBP] (expert-major, NBP = route blocks rounded up to 16,
// padding columns zero); after the scan it holds, for expert e and block b,
// the first sorted row of e's assignments that come from block b.
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float *__restrict__ logits, int T, int E, int k, int tb, int nb, int nbp,
    int32_t *__restrict__ topk_ids, float *__restrict__ topk_w, int32_t *__restrict__ hist)
{
    __shared__ int cnt[kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < E) cnt[tid] = 0;
    // block 0 zeroes the padding columns [nb, nbp) of every expert row
    if (blockIdx.x == 0)
        for (int i = tid; i < E * (nbp - nb); i += kRouteThreads)
            hist[(size_t)(i / (nbp - nb)) * nbp + nb + i % (nbp - nb)] = 0;
    __syncthreads();

    const int t0 = blockIdx.x * tb;
    const int t1 = min(T, t0 + tb);
    for (int t = t0 + wave; t < t1; t += kRouteThreads / kWave) {
        TopK tk;
        wave_topk(logits + (size_t)t * E, E, k, tk);
        // softmax over the selected logits (fp32); slot j lives in lane j % 64
        float ex[4], part = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = lane + 64 * c;
            ex[c] = (j < k) ? expf(tk.logit[c] - tk.lmax) : 0.f;
            part += ex[c];
        }
        const float inv = 1.0f / wave_sum(part);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = lane + 64 * c;
            if (j < k) {
                topk_ids[(size_t)t * k + j] = tk.id[c];
                topk_w[(size_t)t * k + j] = ex[c] * inv;
                atomicAdd(&cnt[tk.id[c]], 1);
            }
        }
    }
    __syncthreads();
    if (tid < E) hist[(size_t)tid * nbp + blockIdx.x] = cnt[tid];
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(
    int32_t *__restrict__ hist, int nbp, int E, int tile_m, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ tile_expert, int32_t *__restrict__ tile_row0,
    int32_t *__restrict__ tile_rows, int32_t *__restrict__ num_tiles)
{
    __shared__ int part[kRouteThreads];
    __shared__ int cnt[kMaxE + 4];
    __shared__ int off[kMaxE + 4];
    __shared__ int tstart[kMaxE + 4];
    const int tid = threadIdx.x;
    // 4 threads per expert, each a contiguous quarter of the (16-padded) blocks,
    // read 4 counts at a time
    const int e = tid >> 2, q = tid & 3;
    const int seg4 = nbp >> 4;  // int4 chunks per quarter
    int4 *row = reinterpret_cast<int4 *>(hist + (size_t)e * nbp) + q * seg4;
    int s = 0;
    if (e < E) {
#pragma unroll 8
        for (int i = 0; i < seg4; ++i) {
            const int4 v = row[i];
            s += v.x + v.y + v.z + v.w;
        }
    }
    part[tid] = s;
    __syncthreads();
    if (tid < kMaxE)
        cnt[tid] = (tid < E) ? part[4 * tid] + part[4 * tid + 1] + part[4 * tid + 2] + part[4 * tid + 3] : 0;
    __syncthreads();
    // exclusive scans over the (at most 256) experts: rows and tiles
    if (tid < kWave) {
        int v[4], nt[4], sv = 0, st = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = cnt[4 * tid + i];
            nt[i] = (v[i] + tile_m - 1) / tile_m;
            sv += v[i];
            st += nt[i];
        }
        int iv = sv, it = st;  // inclusive wave scans
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int a = __shfl_up(iv, o, kWave), b = __shfl_up(it, o, kWave);
            if (tid >= o) { iv += a; it += b; }
        }
        int rv = iv - sv, rt = it - st;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            off[4 * tid + i] = rv;
            tstart[4 * tid + i] = rt;
            rv += v[i];
            rt += nt[i];
        }
        if (tid == kWave - 1) { off[kMaxE] = rv; tstart[kMaxE] = rt; }
    }
    __syncthreads();
    if (tid < E) counts[tid] = cnt[tid];
    if (tid <= E) offsets[tid] = off[tid];
    const int ntiles = tstart[E];
    if (tid == 0) *num_tiles = ntiles;
    // per-block scatter bases (column scan over blocks, in place)
    if (e < E) {
        int base = off[e];
        for (int qq = 0; qq < q; ++qq) base += part[4 * e + qq];
#pragma unroll 8
        for (int i = 0; i < seg4; ++i) {
            const int4 v = row[i];
            int4 o;
            o.x = base; base += v.x;
            o.y = base; base += v.y;
            o.z = base; base += v.z;
            o.w = base; base += v.w;
            row[i] = o;
        }
    }
    // block map: tile i belongs to the expert whose tile range holds it
    for (int i = tid; i < ntiles; i += kRouteThreads) {
        int lo = 0, hi = E - 1;  // last expert with tstart <= i
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int r0 = (i - tstart[lo]) * tile_m;
        tile_expert[i] = lo;
        tile_row0[i] = off[lo] + r0;
        tile_rows[i] = min(tile_m, cnt[lo] - r0);
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t *__restrict__ topk_ids, const int32_t *__restrict__ hist, int nbp, int E,
    int64_t A, int chunk, int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm)
{
    constexpr int kWaves = kRouteThreads / kWave;
    __shared__ int base[kMaxE];
    __shared__ int wcnt[kWaves][kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < E) base[tid] = hist[(size_t)tid * nbp + blockIdx.x];
    const int64_t a0 = (int64_t)blockIdx.x * chunk;
    const int64_t a1 = min(A, a0 + chunk);
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int64_t g = a0; g < a1; g += kRouteThreads) {
        for (int i = tid; i < kWaves * kMaxE; i += kRouteThreads) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int64_t a = g + tid;
        const bool active = a < a1;
        const int e = active ? topk_ids[a] : 0;
        // lanes of this wave holding the same expert (8 id bits, E <= 256)
        uint64_t same = __ballot(active);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bb = __ballot(on);
            same &= on ? bb : ~bb;
        }
        const int rank = __popcll(same & lt_mask);
        if (active && rank == 0) wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (active) {
            int pos = base[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            perm[pos] = (int32_t)a;
            inv_perm[a] = pos;
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w) add += wcnt[w][tid];
            base[tid] += add;
        }
        __syncthreads();
    }
}

hipError_t launch_route(const Plan &p, const float *logits, const moe_routing &r, void *ws,
                        hipStream_t s, EventTrace *tr)
{
    int32_t *hist = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + p.off_hist);
    if (p.route_nb > 0)
        launch(tr, route_topk_kernel, dim3(p.route_nb), dim3(kRouteThreads), 0, s, logits, p.T, p.E,
               p.k, p.route_tb, p.route_nb, p.route_nbp, r.topk_ids, r.topk_w, hist);
    launch(tr, route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, hist, p.route_nbp, p.E,
           p.tile_m, r.counts, r.offsets, r.tile_expert, r.tile_row0, r.tile_rows, r.num_tiles);
    if (p.route_nb > 0)
        launch(tr, route_scatter_kernel, dim3(p.route_nb), dim3(kRouteThreads), 0, s, r.topk_ids,
               (const int32_t *)hist, p.route_nbp, p.E, p.A, p.route_tb * p.k, r.perm, r.inv_perm);
    return hipGetLastError();
}

}  // namespace moe
