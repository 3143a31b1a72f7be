// Host-side internals of the MoE library: derived launch geometry, workspace
// carving and the kernel launchers each .hip file provides.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kRouteThreads = 1024;  // routing kernels: 16 waves per block
constexpr int kMaxE = 256;
// batches of up to kMaxDecodeT tokens (and at most kMaxDecodeAssign token-
// expert assignments) take the matrix-vector kernels of the decode path.
// Measured at d = 2048, E = 256, k = 8, F = Fs = 512 (one weight set, layer
// time): T = 9: 43 us against 82 us on the GEMM path, T = 16: 71 against 90,
// T = 24: 101 against 120, T = 32: 130 against 132.
constexpr int kMaxDecodeT = 32;
constexpr int kMaxDecodeAssign = 512;


// Everything derived from moe_dims that the launchers need.
struct Plan {
    int T, d, E, k, F, Fs, G, tile_m;
    int down_nc;        // requested down-GEMM chain length (0: library picks)
    int64_t A;          // assignments T*k
    int route_tb;       // tokens per route block
    int route_nb;       // route blocks
    int route_nbp;      // route blocks rounded up to a multiple of 16 (histogram row pitch)
    int64_t max_tiles;  // length of the tile arrays
    // workspace carving (byte offsets)
    size_t off_hist, off_hr, off_hs, off_obuf, off_dech, off_gamma, off_router, ws_bytes;
};

// Optional per-kernel timing (measurement entry point): kernel i of a call
// is launched with events[2i] / events[2i+1] as the start / stop events of
// hipExtLaunchKernel, which time exactly that dispatch on its stream.
struct EventTrace {
    hipEvent_t *ev = nullptr;
    int n = 0, i = 0;
    bool take(hipEvent_t *start, hipEvent_t *stop)
    {
        if (!ev || i + 1 >= n) return false;
        *start = ev[i];
        *stop = ev[i + 1];
        i += 2;
        return true;
    }
};

// launch `kernel`, timed by the next event pair of `tr` if there is one
template <typename... KArgs, typename... Args>
inline void launch(EventTrace *tr, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                   hipStream_t s, Args... args)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (tr && tr->take(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// Fills *p; returns MOE_OK or MOE_ERR_SHAPE with a message in *why.
moe_status make_plan(const moe_dims *dims, Plan *p, const char **why);

// ---- route.hip
hipError_t launch_route(const Plan &p, const float *logits, const moe_routing &r, void *ws,
                        hipStream_t s, EventTrace *tr = nullptr);

// ---- router.hip: logits = x W_r (+ bias) from the packed bf16 hi/lo router
int router_epad(int E);                    // experts rounded up to 64 (packed rows)
int router_splits(int T, int d, int E);    // K ranges of the router GEMM
hipError_t launch_router_pack(const float *W, int d, int E, uint16_t *P, hipStream_t s);
hipError_t launch_router(const Plan &p, const uint16_t *x, const uint16_t *P, const float *bias, float *logits,
                         void *ws, hipStream_t s);

// ---- gemm.hip (T >= 2 path)
hipError_t launch_ffn_gemm(const Plan &p, const uint16_t *x, const moe_weights &w,
                           const moe_routing &r, uint16_t *y, void *ws, hipStream_t s,
                           EventTrace *tr = nullptr);

// ---- decode.hip (batches of 1..kMaxDecodeT tokens, two kernels); when
// logits != nullptr the routing is computed in-kernel and written to r,
// else it is read from r.
hipError_t launch_decode(const Plan &p, const float *logits, const uint16_t *x,
                         const moe_weights &w, const moe_routing &r, uint16_t *y, void *ws,
                         hipStream_t s, EventTrace *tr = nullptr);

// ---- attn.hip: decode attention over grouped KV heads (8 query heads per KV head)
// tokens per block (at least `round`, the four slices of a block, and a
// multiple of it or of 32) for `resident` co-resident blocks
int attn_chunk(int Hkv, int L, int resident, int round);
// bound over every device: at most min(1024, ceil(L / 64)) splits per KV head
size_t attn_workspace_bytes(int Hq, int Hkv, int D, int L);
hipError_t launch_gqa_decode(int Hq, int Hkv, int D, int L, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, uint16_t *o, void *ws, hipStream_t s, EventTrace *tr = nullptr);

// ---- dequant.hip
hipError_t launch_dequant(const moe_qmat &m, int rows, int cols, int G, uint16_t *out,
                          hipStream_t s);

}  // namespace moe
