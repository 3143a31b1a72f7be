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
//   2. route_scan_kernel    one block per expert: exclusive scan of the
//                           expert's per-route-block counts (row-relative
//                           scatter bases) and its total;
//   3. route_scatter_kernel one block per route chunk: expert offsets from
//                           the totals (exclusive scan), stable ranks inside
//                           the chunk from wave ballots (a multisplit), then
//                           perm / inv_perm; block 0 also writes counts,
//                           offsets and the tile block map.
//
// Every step is integer-exact and deterministic (LDS integer atomics only
// count, they never order).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// hist layout: [E][NBP] (expert-major, NBP = route blocks rounded up to 16,
// padding columns zero): assignments of expert e in route block b.  bases
// (same layout, written by the scan): the first sorted row of e's
// assignments that come from block b.
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
    constexpr int kStride = kRouteThreads / kWave;
    LogitQuad next;
    if (t0 + wave < t1) next = load_logits(logits + (size_t)(t0 + wave) * E, E);
    for (int t = t0 + wave; t < t1; t += kStride) {
        const LogitQuad cur = next;  // prefetch the wave's next token under this one
        if (t + kStride < t1) next = load_logits(logits + (size_t)(t + kStride) * E, E);
        TopK tk;
        wave_topk(cur, E, k, tk);
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

// One block per expert: exclusive scan of the expert's per-route-block
// counts (its histogram row) -> row-relative scatter bases, and the total.
constexpr int kScanThreads = 128;

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(const int32_t *__restrict__ hist,
                                                                  int32_t *__restrict__ bases,
                                                                  int32_t *__restrict__ totals, int nbp)
{
    __shared__ int wsum[kScanThreads / kWave];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // thread t owns blocks [4 t', 4 t' + 4) for t' = t, t + 128, ... (nbp <= 4096)
    const int4 *row = reinterpret_cast<const int4 *>(hist + (size_t)e * nbp);
    int4 *out = reinterpret_cast<int4 *>(bases + (size_t)e * nbp);
    const int n4 = nbp >> 2;
    int carry = 0;
    for (int c0 = 0; c0 < n4; c0 += kScanThreads) {
        const int c = c0 + tid;
        const int4 v = c < n4 ? row[c] : make_int4(0, 0, 0, 0);
        const int tot = v.x + v.y + v.z + v.w;
        int incl = tot;  // inclusive scan over the block's threads
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int t = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += t;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        int base = before + incl - tot;
        if (c < n4) {
            int4 o;
            o.x = base; base += v.x;
            o.y = base; base += v.y;
            o.z = base; base += v.z;
            o.w = base;
            out[c] = o;
        }
        for (int w = 0; w < kScanThreads / kWave; ++w) carry += wsum[w];
        __syncthreads();
    }
    if (tid == 0) totals[e] = carry;
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t *__restrict__ topk_ids, const int32_t *__restrict__ bases,
    const int32_t *__restrict__ totals, int nbp, int E, int64_t A, int chunk, int tile_m,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ tile_expert, int32_t *__restrict__ tile_row0,
    int32_t *__restrict__ tile_rows, int32_t *__restrict__ num_tiles)
{
    constexpr int kWaves = kRouteThreads / kWave;
    __shared__ int base[kMaxE];
    __shared__ int off[kMaxE + 4];
    __shared__ int tstart[kMaxE + 4];
    __shared__ int wcnt[kWaves][kMaxE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // exclusive scans of the expert totals (rows and tiles) by wave 0
    if (tid < kWave) {
        int v[4], nt[4], sv = 0, st = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * tid + i;
            v[i] = e < E ? totals[e] : 0;
            nt[i] = (v[i] + tile_m - 1) / tile_m;
            sv += v[i];
            st += nt[i];
        }
        int iv = sv, it = st;
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
    if (tid < E) base[tid] = off[tid] + bases[(size_t)tid * nbp + blockIdx.x];
    if (blockIdx.x == 0) {  // histogram, offsets and the tile block map
        if (tid < E) counts[tid] = off[tid + 1] - off[tid];
        if (tid <= E) offsets[tid] = off[tid];
        const int ntiles = tstart[E];
        if (tid == 0) *num_tiles = ntiles;
        for (int i = tid; i < ntiles; i += kRouteThreads) {
            int lo = 0, hi = E - 1;  // last expert with tstart <= i
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (tstart[mid] <= i) lo = mid; else hi = mid - 1;
            }
            const int r0 = (i - tstart[lo]) * tile_m;
            tile_expert[i] = lo;
            tile_row0[i] = off[lo] + r0;
            tile_rows[i] = min(tile_m, off[lo + 1] - off[lo] - r0);
        }
    }
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

// T == 0: the routing outputs of an empty batch
__global__ void route_empty_kernel(int E, int32_t *counts, int32_t *offsets, int32_t *num_tiles)
{
    const int t = threadIdx.x;
    if (t < E) counts[t] = 0;
    if (t <= E) offsets[t] = 0;
    if (t == 0) *num_tiles = 0;
}

hipError_t launch_route(const Plan &p, const float *logits, const moe_routing &r, void *ws,
                        hipStream_t s, EventTrace *tr)
{
    int32_t *hist = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + p.off_hist);
    int32_t *bases = hist + (size_t)p.E * p.route_nbp;
    int32_t *totals = bases + (size_t)p.E * p.route_nbp;
    if (p.route_nb > 0) {
        launch(tr, route_topk_kernel, dim3(p.route_nb), dim3(kRouteThreads), 0, s, logits, p.T, p.E,
               p.k, p.route_tb, p.route_nb, p.route_nbp, r.topk_ids, r.topk_w, hist);
        launch(tr, route_scan_kernel, dim3(p.E), dim3(kScanThreads), 0, s, (const int32_t *)hist, bases,
               totals, p.route_nbp);
        launch(tr, route_scatter_kernel, dim3(p.route_nb), dim3(kRouteThreads), 0, s, r.topk_ids,
               (const int32_t *)bases, (const int32_t *)totals, p.route_nbp, p.E, p.A, p.route_tb * p.k,
               p.tile_m, r.perm, r.inv_perm, r.counts, r.offsets, r.tile_expert, r.tile_row0, r.tile_rows,
               r.num_tiles);
    } else {  // no tokens: empty histogram, zero offsets, no tiles
        launch(tr, route_empty_kernel, dim3(1), dim3(kMaxE + 1), 0, s, p.E, r.counts, r.offsets, r.num_tiles);
    }
    return hipGetLastError();
}

}  // namespace moe
