// C ABI of the MoE layer: host-side validation, workspace carving and the
// launch sequence.  Nothing here touches the device except kernel launches
// on the caller's stream; no host synchronisation, no device-to-host copy
// (the Lily pages attribute a large prefill gain to keeping the routing
// metadata on the GPU with no host round trip: page "Perplexity's Lily Beats
// MLX-LM by 1.35x Running Qwen3.6 on Apple Silicon", section "Prefill
// optimizations", second bullet).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "moe_internal.h"

namespace moe {

static thread_local std::string g_last_error;

static moe_status fail(moe_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

static int pick_tile_m(int64_t A, int E)
{
    const int64_t per_expert = A / (E > 0 ? E : 1);
    if (per_expert <= 32) return 32;
    if (per_expert <= 64) return 64;
    return 128;
}

static bool mult_ok(int v, int G) { return v > 0 && v <= 16384 && v % 64 == 0 && v % G == 0; }

moe_status make_plan(const moe_dims *dm, Plan *p, const char **why)
{
    if (!dm) { *why = "dims is NULL"; return MOE_ERR_ARG; }
    const moe_dims &d = *dm;
    if (d.T < 0 || d.T > (1 << 22)) { *why = "T outside [0, 2^22]"; return MOE_ERR_SHAPE; }
    if (d.E < 1 || d.E > kMaxE) { *why = "E outside [1, 256]"; return MOE_ERR_SHAPE; }
    if (d.k < 1 || d.k > d.E) { *why = "k outside [1, E]"; return MOE_ERR_SHAPE; }
    if ((int64_t)d.T * d.k >= ((int64_t)1 << 31)) { *why = "T*k >= 2^31"; return MOE_ERR_SHAPE; }
    if (d.G != 32 && d.G != 64 && d.G != 128) { *why = "G not in {32, 64, 128}"; return MOE_ERR_SHAPE; }
    if (!mult_ok(d.d, d.G)) { *why = "d must be a positive multiple of 64 and of G, <= 16384"; return MOE_ERR_SHAPE; }
    if (!mult_ok(d.F, d.G)) { *why = "F must be a positive multiple of 64 and of G, <= 16384"; return MOE_ERR_SHAPE; }
    if (!mult_ok(d.Fs, d.G)) { *why = "Fs must be a positive multiple of 64 and of G, <= 16384"; return MOE_ERR_SHAPE; }
    if ((int64_t)d.T * d.d >= ((int64_t)1 << 31) || (int64_t)d.T * d.k * d.F >= ((int64_t)1 << 31) ||
        (int64_t)d.T * d.Fs >= ((int64_t)1 << 31)) {
        *why = "T*d, T*k*F and T*Fs must each be below 2^31";
        return MOE_ERR_SHAPE;
    }
    if (d.tile_m != 0 && d.tile_m != 32 && d.tile_m != 64 && d.tile_m != 128) {
        *why = "tile_m not in {0, 32, 64, 128}";
        return MOE_ERR_SHAPE;
    }
    if (d.down_nc < 0 || d.down_nc > 64) { *why = "down_nc outside [0, 64]"; return MOE_ERR_SHAPE; }
    if (d.down_nc > 1) {
        const int nk = d.F / 64;
        if (d.d % 256 != 0 || d.F != d.Fs || nk < 2 || (nk & (nk - 1)) != 0 || (d.d / 256) % d.down_nc != 0) {
            *why = "down_nc > 1 needs d a multiple of 256, F = Fs = 64 * 2^n (n >= 1) and down_nc dividing d/256";
            return MOE_ERR_SHAPE;
        }
    }
    p->T = d.T; p->d = d.d; p->E = d.E; p->k = d.k; p->F = d.F; p->Fs = d.Fs; p->G = d.G;
    p->down_nc = d.down_nc;
    p->A = (int64_t)d.T * d.k;
    p->tile_m = d.tile_m ? d.tile_m : pick_tile_m(p->A, d.E);
    // route chunks: 16 tokens per route block (one per wave of the top-k kernel)
    const int tb = 16;
    p->route_tb = tb;
    p->route_nb = (d.T + tb - 1) / tb;
    p->route_nbp = (p->route_nb + 15) & ~15;
    p->max_tiles = (p->A + p->tile_m - 1) / p->tile_m + (p->A < d.E ? p->A : d.E);
    const int Fmax = d.F > d.Fs ? d.F : d.Fs;
    size_t off = 0;
    p->off_hist = off; off = align_up(off + ((size_t)2 * d.E * p->route_nbp + d.E) * 4);  // counts, bases, totals
    p->off_hr = off;   off = align_up(off + (size_t)p->A * d.F * 2);
    p->off_hs = off;   off = align_up(off + (size_t)d.T * d.Fs * 2);
    p->off_obuf = off; off = align_up(off + (size_t)(p->A + d.T) * d.d * 2);
    // decode path (batches of at most kMaxDecodeT tokens): h per token and slot,
    // the shared expert's gate value per token
    const int td = d.T < 1 ? 1 : (d.T < kMaxDecodeT ? d.T : kMaxDecodeT);
    p->off_dech = off; off = align_up(off + (size_t)td * (d.k + 1) * Fmax * 4);
    p->off_gamma = off; off = align_up(off + (size_t)kMaxDecodeT * 4);
    // router GEMM: partial logits of its K ranges (only when it splits K)
    const int ks = router_splits(d.T, d.d, d.E);
    p->off_router = off; off = align_up(off + (ks > 1 ? (size_t)ks * d.T * d.E * 4 : 0));
    p->ws_bytes = off;
    return MOE_OK;
}

// non-empty arrays must be non-null and 16-byte aligned
static bool ptr_ok(const void *ptr, size_t nbytes)
{
    if (nbytes == 0) return true;
    return ptr && (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

static bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!na || !nb || !a || !b) return false;
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

static moe_status check_qmat(const moe_qmat &m, const char *name, int64_t rows, int cols, int G)
{
    if (!ptr_ok(m.q, (size_t)rows * cols / 2) || !ptr_ok(m.s, (size_t)rows * (cols / G) * 2) ||
        !ptr_ok(m.b, (size_t)rows * (cols / G) * 2))
        return fail(MOE_ERR_ARG, "weight %s: null or misaligned pointer", name);
    return MOE_OK;
}

static moe_status check_weights(const Plan &p, const moe_weights *w)
{
    if (!w) return fail(MOE_ERR_ARG, "weights struct is NULL");
    moe_status st;
    if ((st = check_qmat(w->gate, "gate", (int64_t)p.E * p.F, p.d, p.G))) return st;
    if ((st = check_qmat(w->up, "up", (int64_t)p.E * p.F, p.d, p.G))) return st;
    if ((st = check_qmat(w->down, "down", (int64_t)p.E * p.d, p.F, p.G))) return st;
    if ((st = check_qmat(w->sgate, "sgate", p.Fs, p.d, p.G))) return st;
    if (w->shared_gate && (reinterpret_cast<uintptr_t>(w->shared_gate) & 15u))
        return fail(MOE_ERR_ARG, "shared_gate: misaligned pointer");
    if ((st = check_qmat(w->sup, "sup", p.Fs, p.d, p.G))) return st;
    if ((st = check_qmat(w->sdown, "sdown", p.d, p.Fs, p.G))) return st;
    return MOE_OK;
}

static moe_status check_routing(const Plan &p, const moe_routing *r)
{
    if (!r) return fail(MOE_ERR_ARG, "routing struct is NULL");
    const size_t A4 = (size_t)p.A * 4, MT4 = (size_t)p.max_tiles * 4;
    if (!ptr_ok(r->topk_ids, A4) || !ptr_ok(r->topk_w, A4) || !ptr_ok(r->counts, (size_t)p.E * 4) ||
        !ptr_ok(r->offsets, (size_t)(p.E + 1) * 4) || !ptr_ok(r->perm, A4) || !ptr_ok(r->inv_perm, A4) ||
        !ptr_ok(r->tile_expert, MT4) || !ptr_ok(r->tile_row0, MT4) || !ptr_ok(r->tile_rows, MT4) ||
        !ptr_ok(r->num_tiles, 4))
        return fail(MOE_ERR_ARG, "routing: null or misaligned pointer");
    return MOE_OK;
}

static moe_status common(const moe_dims *dims, Plan *p, void *ws, size_t ws_bytes)
{
    const char *why = "";
    moe_status st = make_plan(dims, p, &why);
    if (st != MOE_OK) return fail(st, "%s", why);
    if (ws_bytes < p->ws_bytes)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p->ws_bytes);
    if (!ptr_ok(ws, p->ws_bytes)) return fail(MOE_ERR_ARG, "workspace: null or misaligned pointer");
    return MOE_OK;
}

static moe_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

MOE_API int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API int32_t moe_tile_m(const moe_dims *dims)
{
    Plan p;
    const char *why;
    return make_plan(dims, &p, &why) == MOE_OK ? p.tile_m : 0;
}

MOE_API size_t moe_max_tiles(const moe_dims *dims)
{
    Plan p;
    const char *why;
    return make_plan(dims, &p, &why) == MOE_OK ? (size_t)p.max_tiles : 0;
}

MOE_API size_t moe_workspace_bytes(const moe_dims *dims)
{
    Plan p;
    const char *why;
    return make_plan(dims, &p, &why) == MOE_OK ? p.ws_bytes : 0;
}

MOE_API moe_status moe_route(const moe_dims *dims, const float *logits, const moe_routing *out,
                             void *ws, size_t ws_bytes, void *stream)
{
    Plan p;
    moe_status st = common(dims, &p, ws, ws_bytes);
    if (st) return st;
    if (!ptr_ok(logits, (size_t)p.T * p.E * 4)) return fail(MOE_ERR_ARG, "logits: null or misaligned pointer");
    if ((st = check_routing(p, out))) return st;
    (void)hipGetLastError();
    return hip_status(launch_route(p, logits, *out, ws, (hipStream_t)stream), "moe_route launch");
}

MOE_API size_t moe_router_packed_bytes(const moe_dims *dims)
{
    Plan p;
    const char *why;
    if (make_plan(dims, &p, &why) != MOE_OK) return 0;
    return (size_t)2 * router_epad(p.E) * p.d * 2;
}

MOE_API moe_status moe_router_pack(const moe_dims *dims, const float *w_router, uint16_t *packed, void *stream)
{
    Plan p;
    const char *why = "";
    moe_status st = make_plan(dims, &p, &why);
    if (st != MOE_OK) return fail(st, "%s", why);
    const size_t wb = (size_t)p.d * p.E * 4, pb = (size_t)2 * router_epad(p.E) * p.d * 2;
    if (!ptr_ok(w_router, wb)) return fail(MOE_ERR_ARG, "w_router: null or misaligned pointer");
    if (!ptr_ok(packed, pb)) return fail(MOE_ERR_ARG, "packed: null or misaligned pointer");
    if (overlap(w_router, wb, packed, pb)) return fail(MOE_ERR_ARG, "w_router and packed overlap");
    (void)hipGetLastError();
    return hip_status(launch_router_pack(w_router, p.d, p.E, packed, (hipStream_t)stream), "moe_router_pack launch");
}

MOE_API moe_status moe_route_x(const moe_dims *dims, const uint16_t *x, const uint16_t *packed, const float *bias,
                               float *logits, const moe_routing *out, void *ws, size_t ws_bytes, void *stream)
{
    Plan p;
    moe_status st = common(dims, &p, ws, ws_bytes);
    if (st) return st;
    const size_t xb = (size_t)p.T * p.d * 2, lb = (size_t)p.T * p.E * 4;
    const size_t pb = (size_t)2 * router_epad(p.E) * p.d * 2;
    if (!ptr_ok(x, xb)) return fail(MOE_ERR_ARG, "x: null or misaligned pointer");
    if (!ptr_ok(packed, pb)) return fail(MOE_ERR_ARG, "packed: null or misaligned pointer");
    if (!ptr_ok(logits, lb)) return fail(MOE_ERR_ARG, "logits: null or misaligned pointer");
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)) return fail(MOE_ERR_ARG, "bias: misaligned pointer");
    if (overlap(x, xb, logits, lb) || overlap(packed, pb, logits, lb))
        return fail(MOE_ERR_ARG, "logits overlaps x or packed");
    if ((st = check_routing(p, out))) return st;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_router(p, x, packed, bias, logits, ws, s);
    if (e == hipSuccess) e = launch_route(p, logits, *out, ws, s);
    return hip_status(e, "moe_route_x launch");
}

// Batches of 1..kMaxDecodeT tokens run the matrix-vector kernels of the
// decode path (each token streams its experts' rows; no tiles to fill).
static bool decode_batch(const Plan &p)
{
    return p.T >= 1 && p.T <= kMaxDecodeT && p.A <= kMaxDecodeAssign;
}

MOE_API moe_status moe_ffn(const moe_dims *dims, const uint16_t *x, const moe_weights *w,
                           const moe_routing *r, uint16_t *y, void *ws, size_t ws_bytes, void *stream)
{
    Plan p;
    moe_status st = common(dims, &p, ws, ws_bytes);
    if (st) return st;
    const size_t xb = (size_t)p.T * p.d * 2;
    if (!ptr_ok(x, xb) || !ptr_ok(y, xb)) return fail(MOE_ERR_ARG, "x / y: null or misaligned pointer");
    if (overlap(x, xb, y, xb)) return fail(MOE_ERR_ARG, "x and y overlap");
    if ((st = check_weights(p, w)) || (st = check_routing(p, r))) return st;
    if (p.T == 0) return MOE_OK;
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (decode_batch(p))
        e = launch_decode(p, nullptr, x, *w, *r, y, ws, s);
    else
        e = launch_ffn_gemm(p, x, *w, *r, y, ws, s);
    return hip_status(e, "moe_ffn launch");
}

static int layer_kernels(const Plan &p)
{
    if (decode_batch(p)) return 2;       // decode gate/up, decode down
    if (p.T == 0) return 1;              // empty routing
    return 3 + 3;                        // route topk, scan, scatter; gate/up, down, combine
}

// the layer's pointer arguments (everything but the workspace)
static moe_status check_layer_args(const Plan &p, const float *logits, const uint16_t *x, const moe_weights *w,
                                   const moe_routing *out, const uint16_t *y)
{
    moe_status st;
    const size_t xb = (size_t)p.T * p.d * 2;
    if (!ptr_ok(logits, (size_t)p.T * p.E * 4)) return fail(MOE_ERR_ARG, "logits: null or misaligned pointer");
    if (!ptr_ok(x, xb) || !ptr_ok(y, xb)) return fail(MOE_ERR_ARG, "x / y: null or misaligned pointer");
    if (overlap(x, xb, y, xb)) return fail(MOE_ERR_ARG, "x and y overlap");
    if ((st = check_weights(p, w)) || (st = check_routing(p, out))) return st;
    return MOE_OK;
}

// route + ffn on validated arguments
static moe_status launch_layer(const Plan &p, const float *logits, const uint16_t *x, const moe_weights *w,
                               const moe_routing *out, uint16_t *y, void *ws, void *stream, EventTrace *tr)
{
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e;
    if (decode_batch(p)) {
        e = launch_decode(p, logits, x, *w, *out, y, ws, s, tr);
    } else {
        e = launch_route(p, logits, *out, ws, s, tr);
        if (e == hipSuccess && p.T > 0) e = launch_ffn_gemm(p, x, *w, *out, y, ws, s, tr);
    }
    return hip_status(e, "moe_layer launch");
}

static moe_status layer_impl(const moe_dims *dims, const float *logits, const uint16_t *x,
                             const moe_weights *w, const moe_routing *out, uint16_t *y, void *ws,
                             size_t ws_bytes, void *stream, EventTrace *tr)
{
    Plan p;
    moe_status st = common(dims, &p, ws, ws_bytes);
    if (st) return st;
    if ((st = check_layer_args(p, logits, x, w, out, y))) return st;
    if (tr && tr->n < 2 * layer_kernels(p))
        return fail(MOE_ERR_ARG, "need %d events, got %d", 2 * layer_kernels(p), tr->n);
    return launch_layer(p, logits, x, w, out, y, ws, stream, tr);
}

// ---- allocation-free entry point ------------------------------------------------
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES
// that the code object brings with it (each GPU the library runs on holds its
// own copy until the process ends).  Its device address is looked up once per
// device with that device current and kept; the array's name is never used in
// host code as an address.  No kernel needs any of it to start at zero: every
// element a kernel reads was written earlier in the same call.

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// the current device's copy of `scratch` (nullptr and *why set on failure)
static void *scratch_address(const char **why)
{
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *why = "no current HIP device (or device index >= 64)";
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *why = hipGetErrorString(e);
            return nullptr;
        }
        addr[dev] = ptr;
    }
    return addr[dev];
}

MOE_API moe_status moe_layer(const moe_dims *dims, const float *logits, const uint16_t *x,
                             const moe_weights *w, const moe_routing *out, uint16_t *y, void *ws,
                             size_t ws_bytes, void *stream)
{
    return layer_impl(dims, logits, x, w, out, y, ws, ws_bytes, stream, nullptr);
}

MOE_API moe_status moe_layer_noalloc(const moe_dims *dims, const float *logits, const uint16_t *x,
                                     const moe_weights *w, const moe_routing *out, uint16_t *y, void *stream)
{
    Plan p;
    const char *why = "";
    moe_status st = make_plan(dims, &p, &why);
    if (st != MOE_OK) return fail(st, "%s", why);
    if (p.ws_bytes > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "these dims need %zu bytes of workspace; the allocation-free entry point holds %zu "
                    "(call moe_layer with a caller-owned workspace)",
                    p.ws_bytes, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    if ((st = check_layer_args(p, logits, x, w, out, y))) return st;
    void *ws = scratch_address(&why);
    if (!ws) return fail(MOE_ERR_HIP, "scratch address: %s", why);
    (void)hipGetLastError();
    return launch_layer(p, logits, x, w, out, y, ws, stream, nullptr);
}

MOE_API int32_t moe_layer_kernels(const moe_dims *dims)
{
    Plan p;
    const char *why;
    return make_plan(dims, &p, &why) == MOE_OK ? layer_kernels(p) : 0;
}

MOE_API moe_status moe_layer_timed(const moe_dims *dims, const float *logits, const uint16_t *x,
                                   const moe_weights *w, const moe_routing *out, uint16_t *y,
                                   void *ws, size_t ws_bytes, void *stream, void *const *events,
                                   int32_t n_events)
{
    if (!events) return fail(MOE_ERR_ARG, "events is NULL");
    EventTrace tr;
    tr.ev = reinterpret_cast<hipEvent_t *>(const_cast<void **>(events));
    tr.n = n_events;
    return layer_impl(dims, logits, x, w, out, y, ws, ws_bytes, stream, &tr);
}

// ---- decode attention over grouped KV heads

static bool attn_dims_ok(const moe_attn_dims *d, const char **why)
{
    if (!d) { *why = "dims is NULL"; return false; }
    if (d->Hkv < 1 || d->Hkv > 128 || d->Hq != 8 * d->Hkv) { *why = "need Hq = 8 * Hkv, 1 <= Hkv <= 128"; return false; }
    if (d->D != 64 && d->D != 128 && d->D != 256) { *why = "D not in {64, 128, 256}"; return false; }
    if (d->L < 1 || d->L > (1 << 24)) { *why = "L outside [1, 2^24]"; return false; }
    return true;
}

MOE_API size_t moe_gqa_workspace_bytes(const moe_attn_dims *dims)
{
    const char *why;
    if (!attn_dims_ok(dims, &why)) return 0;
    return attn_workspace_bytes(dims->Hq, dims->Hkv, dims->D, dims->L);
}

static moe_status gqa_impl(const moe_attn_dims *dims, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           uint16_t *o, void *ws, size_t ws_bytes, void *stream, EventTrace *tr)
{
    const char *why;
    if (!attn_dims_ok(dims, &why)) return fail(dims ? MOE_ERR_SHAPE : MOE_ERR_ARG, "%s", why);
    const moe_attn_dims &d = *dims;
    const size_t qb = (size_t)d.Hq * d.D * 2, kvb = (size_t)d.Hkv * d.L * d.D * 2;
    const size_t need = attn_workspace_bytes(d.Hq, d.Hkv, d.D, d.L);
    if (!ptr_ok(q, qb)) return fail(MOE_ERR_ARG, "q: null or misaligned pointer");
    if (!ptr_ok(k, kvb)) return fail(MOE_ERR_ARG, "k: null or misaligned pointer");
    if (!ptr_ok(v, kvb)) return fail(MOE_ERR_ARG, "v: null or misaligned pointer");
    if (!ptr_ok(o, qb)) return fail(MOE_ERR_ARG, "o: null or misaligned pointer");
    if (!ptr_ok(ws, need)) return fail(MOE_ERR_ARG, "workspace: null or misaligned pointer");
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    if (overlap(o, qb, q, qb) || overlap(o, qb, k, kvb) || overlap(o, qb, v, kvb) || overlap(o, qb, ws, need) ||
        overlap(ws, need, q, qb) || overlap(ws, need, k, kvb) || overlap(ws, need, v, kvb))
        return fail(MOE_ERR_ARG, "o or the workspace overlaps another array");
    return hip_status(launch_gqa_decode(d.Hq, d.Hkv, d.D, d.L, q, k, v, o, ws, (hipStream_t)stream, tr),
                      "moe_gqa_decode launch");
}

MOE_API moe_status moe_gqa_decode(const moe_attn_dims *dims, const uint16_t *q, const uint16_t *k,
                                  const uint16_t *v, uint16_t *o, void *ws, size_t ws_bytes, void *stream)
{
    return gqa_impl(dims, q, k, v, o, ws, ws_bytes, stream, nullptr);
}

MOE_API moe_status moe_gqa_decode_timed(const moe_attn_dims *dims, const uint16_t *q, const uint16_t *k,
                                        const uint16_t *v, uint16_t *o, void *ws, size_t ws_bytes,
                                        void *stream, void *const *events, int32_t n_events)
{
    if (!events || n_events < 4) return fail(MOE_ERR_ARG, "events: need 4 event handles");
    EventTrace tr;
    tr.ev = reinterpret_cast<hipEvent_t *>(const_cast<void **>(events));
    tr.n = n_events;
    return gqa_impl(dims, q, k, v, o, ws, ws_bytes, stream, &tr);
}

MOE_API moe_status moe_dequant(const moe_qmat *m, int32_t rows, int32_t cols, int32_t G,
                               uint16_t *out_bf16, void *stream)
{
    if (!m) return fail(MOE_ERR_ARG, "qmat is NULL");
    if (G != 32 && G != 64 && G != 128) return fail(MOE_ERR_SHAPE, "G not in {32, 64, 128}");
    if (rows < 0 || cols <= 0 || cols % 32 || cols % G) return fail(MOE_ERR_SHAPE, "bad rows / cols");
    const size_t n = (size_t)rows * cols;
    if (!ptr_ok(m->q, n / 2) || !ptr_ok(m->s, n / G * 2) || !ptr_ok(m->b, n / G * 2) ||
        !ptr_ok(out_bf16, n * 2))
        return fail(MOE_ERR_ARG, "null or misaligned pointer");
    (void)hipGetLastError();
    return hip_status(launch_dequant(*m, rows, cols, G, out_bf16, (hipStream_t)stream), "moe_dequant launch");
}

MOE_API const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

MOE_API const char *moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
