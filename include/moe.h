/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts FFN layer.
 *
 * The layer is the one the Lily pages describe for Qwen3.6-35B-A3B: every
 * token is sent to the k best of E experts plus one always-on shared expert
 * (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
 * Silicon", section "What Lily actually does"); the weights are groupwise
 * affine 4-bit codes that are decoded tile by tile inside the matrix kernels
 * and never written out as a full bf16 copy (same page, section "Prefill
 * optimizations", first bullet); the expert grouping is a histogram, a prefix
 * scan, a scatter and a block-map build that stay on the GPU with no host
 * round trip (same section, second bullet); prefill runs matrix-core GEMMs,
 * batch-1 decode runs bandwidth-bound matrix-vector kernels (same page,
 * section "Why prefill and decode get different treatment").
 *
 * Conventions
 *  - Pointers are DEVICE pointers unless a comment says otherwise; bf16 values
 *    travel as uint16_t bit patterns.  Every array is dense, row-major, and
 *    must be 16-byte aligned.  Inputs must not alias outputs.
 *  - The caller owns every buffer (inputs, outputs, workspace).  The library
 *    allocates nothing and keeps no state between calls beyond a per-device
 *    cache of the decode-attention kernels' co-resident block counts (queried
 *    once) and the scratch array of moe_layer_noalloc; it is safe to call
 *    from several host threads on different streams (except that calls of
 *    moe_layer_noalloc that overlap on one GPU share its scratch array).
 *  - All compute calls are asynchronous on `stream` (a hipStream_t, or NULL
 *    for the default stream).  No call synchronises the host or copies data
 *    to the host.  Arguments are validated on the host before anything is
 *    enqueued: on a non-OK status nothing was enqueued and moe_last_error()
 *    tells why.  Faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Results are deterministic: identical inputs give identical bits (for
 *    moe_gqa_decode, on one kind of GPU: its split count follows the device).
 *
 * Weight layout (the pages give the format only as "groupwise affine 4-bit";
 * the layout is this library's choice): a matrix W[N_out][K_in] is
 *    q[N_out][K_in/2]  uint8  -- element 2m in the low nibble of byte m,
 *                                element 2m+1 in the high nibble;
 *    s[N_out][K_in/G]  bf16   -- scale of each group of G input elements;
 *    b[N_out][K_in/G]  bf16   -- bias of the group;
 * and w[n][i] = s[n][i/G] * q[n][i] + b[n][i/G].  Routed experts are stacked
 * expert-major: gate and up are [E][F][d], down is [E][d][F]; the shared
 * expert has gate/up [Fs][d] and down [d][Fs].
 *
 * Layer math: for token t with top-k experts e_j and routing weights w_j,
 *    y[t] = sum_j w_j * FFN_{e_j}(x[t]) + FFN_shared(x[t]),
 *    FFN(x) = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + e^-z).
 * Top-k order: larger logit first, equal logits -> lower expert id (-0 and +0
 * are equal); w_j = softmax over the k selected logits.  Logits must be
 * finite.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: route / ffn / layer; 2: optional gated shared expert (moe_weights.shared_gate);
 * 3: moe_router_pack / moe_route_x / moe_router_packed_bytes;
 * 4: moe_dims.down_nc (explicit schedule field, no environment variable);
 * 5: moe_gqa_decode / moe_gqa_decode_timed / moe_gqa_workspace_bytes. */
#define MOE_ABI_VERSION 5

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,       /* null or misaligned pointer, aliasing, bad enum */
    MOE_ERR_SHAPE = 2,     /* dimension outside the supported range */
    MOE_ERR_WORKSPACE = 3, /* ws_bytes below moe_workspace_bytes() */
    MOE_ERR_HIP = 4        /* a HIP launch failed */
} moe_status;

/* Layer shape.  Supported: 0 <= T <= 2^22 (T*k < 2^31); 1 <= k <= E <= 256;
 * G in {32, 64, 128}; d, F and Fs positive multiples of 64 and of G, at most
 * 16384; T*d, T*k*F and T*Fs below 2^31 (each activation matrix of the
 * prefill path under 4 GiB, addressed with 32-bit offsets).
 * tile_m: height of a block-map tile, one of {32, 64, 128}, or 0 to let the
 * library pick from T*k/E (moe_tile_m reports the choice).
 * down_nc: schedule of the prefill down GEMM, 0 to let the library pick, or
 * the number of consecutive 256-column blocks of a tile one workgroup runs as
 * one pipeline: 1, or a divisor of d/256 when d is a multiple of 256 and
 * F = Fs = 64 * 2^n (n >= 1); other values are MOE_ERR_SHAPE.  It changes the
 * schedule only, never the result (bit-identical y for every value); the
 * decode path ignores it. */
typedef struct {
    int32_t T, d, E, k, F, Fs, G, tile_m;
    int32_t down_nc;
} moe_dims;

/* One packed matrix (see the layout above). */
typedef struct {
    const uint8_t *q;
    const uint16_t *s;
    const uint16_t *b;
} moe_qmat;

typedef struct {
    moe_qmat gate, up, down;    /* routed: [E][F][d], [E][F][d], [E][d][F] */
    moe_qmat sgate, sup, sdown; /* shared: [Fs][d], [Fs][d], [d][Fs] */
    /* Optional gate of the shared expert, bf16 [d], 16-byte aligned, or NULL
     * (weight 1).  With it the shared expert's output for token t is scaled
     * by sigmoid(x_t . shared_gate), the dot product accumulated in fp32.
     * The pages name an always-on shared expert and nothing more; the gated
     * form is an optional variant (ABI version 2). */
    const uint16_t *shared_gate;
} moe_weights;

/* Routing results (outputs of moe_route, inputs of moe_ffn).  Assignment
 * a = t*k + j is the j-th expert choice of token t.
 *   topk_ids[T][k]   expert of each assignment, in top-k order;
 *   topk_w[T][k]     routing weight (fp32) of each assignment;
 *   counts[E]        assignments per expert (the histogram);
 *   offsets[E+1]     exclusive prefix sum of counts, offsets[E] = T*k;
 *   perm[T*k]        assignments sorted by expert, ascending a inside one
 *                    expert (stable scatter): sorted row p holds perm[p];
 *   inv_perm[T*k]    inverse permutation: inv_perm[perm[p]] = p;
 *   tile_expert, tile_row0, tile_rows [moe_max_tiles()]: the block map --
 *                    for each expert in id order, tiles of tile_m consecutive
 *                    sorted rows (the last one shorter), as (expert, first
 *                    sorted row, row count); entries past num_tiles are
 *                    unspecified;
 *   num_tiles[1]     number of tiles (written on the device). */
typedef struct {
    int32_t *topk_ids;
    float *topk_w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv_perm;
    int32_t *tile_expert;
    int32_t *tile_row0;
    int32_t *tile_rows;
    int32_t *num_tiles;
} moe_routing;

/* MOE_ABI_VERSION of the loaded library. */
MOE_API int32_t moe_abi_version(void);

/* Host-only, pure.  Effective tile height for these dims (resolves
 * tile_m == 0), or 0 if the dims are invalid. */
MOE_API int32_t moe_tile_m(const moe_dims *dims);

/* Host-only, pure.  Length of the tile_* arrays: ceil(T*k/tile_m) +
 * min(E, T*k), an upper bound of the tile count; 0 for invalid dims. */
MOE_API size_t moe_max_tiles(const moe_dims *dims);

/* Host-only, pure.  Bytes of device workspace moe_route / moe_ffn /
 * moe_layer need for these dims; 0 for invalid dims. */
MOE_API size_t moe_workspace_bytes(const moe_dims *dims);

/* Routing on the GPU: logits fp32 [T][E] (device) -> every field of *out.
 * Top-k and weights, the expert histogram, the exclusive prefix scan, the
 * stable scatter and the block map (Lily pages, section "Prefill
 * optimizations": histogram, prefix scan, scatter, block-map build in one
 * submission).  `out` is a host pointer to a struct of device pointers. */
MOE_API moe_status moe_route(const moe_dims *dims, const float *logits, const moe_routing *out,
                     void *ws, size_t ws_bytes, void *stream);

/* Host-only, pure.  Bytes of the packed router that moe_router_pack writes
 * and moe_route_x reads: 2 * roundup(E, 64) * d bf16 values; 0 for invalid
 * dims. */
MOE_API size_t moe_router_packed_bytes(const moe_dims *dims);

/* Router weights for moe_route_x, once per weight set: w_router fp32 [d][E]
 * (device) -> packed (device, moe_router_packed_bytes): the bf16 pair
 * hi = bf16(W), lo = bf16(W - hi), expert-major [2][roundup(E,64)][d], padding
 * rows zero.  x W = x hi + x lo up to 2^-17 |W| per weight.  Asynchronous on
 * `stream`; the caller owns both buffers. */
MOE_API moe_status moe_router_pack(const moe_dims *dims, const float *w_router, uint16_t *packed, void *stream);

/* Routing from the activations: logits fp32 [T][E] = x W_r (+ bias) on the
 * bf16 matrix cores from the packed router (x bf16 [T][d]; bias fp32 [E] or
 * NULL; fp32 accumulation, deterministic), written to `logits` (device,
 * caller-owned), then the routing of moe_route on those logits into *out.
 * The router computes each token's scores against every expert before its
 * experts are picked (page "Perplexity's Lily Beats MLX-LM by 1.35x Running
 * Qwen3.6 on Apple Silicon", section "What Lily actually does"). */
MOE_API moe_status moe_route_x(const moe_dims *dims, const uint16_t *x, const uint16_t *packed, const float *bias,
                               float *logits, const moe_routing *out, void *ws, size_t ws_bytes, void *stream);

/* Expert FFN: x bf16 [T][d] + weights + routing (as produced by moe_route)
 * -> y bf16 [T][d].  Grouped GEMMs over the block map with the 4-bit weights
 * decoded inside the kernel, or, for small batches (1 <= T <= 32 and T*k <= 512:
 * single-token decode and the pages' few-token verify passes, section "What
 * failed" of "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
 * Silicon"), matrix-vector kernels that stream each token's expert rows.
 * `w` and `r` are host pointers to structs of device pointers; ws must not
 * be shared with a concurrently running call.  The routing arrays are read as
 * moe_route writes them; an out-of-range expert id, tile entry or perm value
 * is clamped into range (a corrupt routing gives wrong y, never an access
 * outside the caller's arrays). */
MOE_API moe_status moe_ffn(const moe_dims *dims, const uint16_t *x, const moe_weights *w,
                   const moe_routing *r, uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* The whole layer: moe_route followed by moe_ffn, enqueued as one sequence
 * on `stream` with no host round trip between the routing and the experts
 * (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple
 * Silicon", section "Prefill optimizations", second bullet: the routing
 * metadata is built on the GPU inside the same submission as the expert
 * matrices; section "What Lily actually does": k routed experts plus the
 * shared expert per token).  For small batches (1 <= T <= 32 and T*k <= 512)
 * the routing is computed inside the matrix-vector kernels (every field of
 * *out is still written, identical to moe_route's). */
MOE_API moe_status moe_layer(const moe_dims *dims, const float *logits, const uint16_t *x,
                     const moe_weights *w, const moe_routing *out, uint16_t *y,
                     void *ws, size_t ws_bytes, void *stream);

/* Bytes of the device scratch array behind moe_layer_noalloc: dims with
 * moe_workspace_bytes() above this are rejected by it (32 MiB: T = 512 at
 * d = 2048, E = 256, k = 8, F = Fs = 512 needs about 24 MB). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library's code object (one per GPU,
 * held until the process ends); the call itself allocates nothing.  The
 * caller still owns x, y, the weights and every routing array, exactly as in
 * moe_layer, and gets identical results.  Dims whose moe_workspace_bytes()
 * exceed MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE with nothing
 * enqueued.  Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (different streams, host threads) race and must be
 * serialised by the caller.  Asynchronous on `stream`. */
MOE_API moe_status moe_layer_noalloc(const moe_dims *dims, const float *logits, const uint16_t *x,
                                     const moe_weights *w, const moe_routing *out, uint16_t *y,
                                     void *stream);

/* Host-only, pure.  Number of kernels one moe_layer call launches for these
 * dims, in launch order: small batches (1 <= T <= 32, T*k <= 512): decode
 * gate/up (with routing), decode down; larger T: route top-k, route scan,
 * route scatter, gate/up GEMM, down GEMM (routed and shared rows), combine;
 * T == 0: empty routing.  0 for invalid dims. */
MOE_API int32_t moe_layer_kernels(const moe_dims *dims);

/* Measurement form of moe_layer: identical work; kernel i is launched with
 * events[2i] and events[2i+1] (hipEvent_t handles created by the caller) as
 * the start and stop events of that one dispatch (hipExtLaunchKernel), so
 * their elapsed time is kernel i's execution time on `stream`.  Needs
 * n_events >= 2 * moe_layer_kernels() (else MOE_ERR_ARG, nothing enqueued).
 * Not for use under stream capture. */
MOE_API moe_status moe_layer_timed(const moe_dims *dims, const float *logits, const uint16_t *x,
                                   const moe_weights *w, const moe_routing *out, uint16_t *y,
                                   void *ws, size_t ws_bytes, void *stream, void *const *events,
                                   int32_t n_events);

/* Decode a packed [rows][cols] matrix to bf16 [rows][cols] with the same
 * device routine the GEMM kernels use: bf16_rne(fp32_rne(s*q + b)), the
 * groupwise affine 4-bit format (page "Perplexity Open Sources Lily: Rust &
 * Metal Engine for Qwen3.6", paragraph on the model) expanded to the bf16
 * values the matrix kernels multiply (page "Perplexity's Lily Beats MLX-LM by
 * 1.35x Running Qwen3.6 on Apple Silicon", section "Prefill optimizations",
 * first bullet: tiles are unpacked on chip right before the multiply).  A
 * test and inspection export; the layer itself never materialises this
 * array.  Needs cols a multiple of 32 and of G, G in {32, 64, 128}; out_bf16
 * is caller-owned, rows*cols bf16; invalid arguments return a status with
 * nothing enqueued. */
MOE_API moe_status moe_dequant(const moe_qmat *m, int32_t rows, int32_t cols, int32_t G,
                       uint16_t *out_bf16, void *stream);

/* Static description of a status code. */
MOE_API const char *moe_status_string(moe_status s);

/* Detail of the last non-OK status returned on this host thread. */
MOE_API const char *moe_last_error(void);

/* ---- Decode attention over grouped KV heads (a second decode workload) -----
 * One decode token attends over L cached tokens, and eight query heads share
 * one KV head (page "Perplexity's Lily Beats MLX-LM by 1.35x Running Qwen3.6
 * on Apple Silicon", section "Decode optimizations"); every cached K and V
 * row is read from memory once for its eight heads.  The pages do not write
 * the formula; this is scaled dot-product attention:
 *   o[h] = sum_t softmax_t(q[h] . k[g][t] / sqrt(D)) v[g][t],  g = h / 8,
 * fp32 arithmetic from bf16 inputs (finite: non-finite q, k or v are outside
 * the contract), o rounded to bf16 (nearest even).
 * Supported: Hkv >= 1, Hq = 8 * Hkv, Hq <= 1024; D in {64, 128, 256};
 * 1 <= L <= 2^24. */
typedef struct {
    int32_t Hq, Hkv, D, L;
} moe_attn_dims;

/* Host-only, pure.  Workspace bytes of moe_gqa_decode (fp32 partial results
 * of the context splits); 0 for invalid dims. */
MOE_API size_t moe_gqa_workspace_bytes(const moe_attn_dims *dims);

/* q bf16 [Hq][D]; k, v bf16 [Hkv][L][D] (one row per cached token); o bf16
 * [Hq][D], caller-owned; ws: moe_gqa_workspace_bytes() bytes, any contents
 * (fully rewritten by each call).  Two kernels on `stream` (context splits,
 * then their combination in a fixed order).  The split count follows the
 * device (its co-resident block count), so results are bit-identical from
 * call to call on one kind of GPU and may differ in the last bits between
 * kinds.  o must not overlap the inputs or ws.  Invalid arguments return a
 * status with nothing enqueued. */
MOE_API moe_status moe_gqa_decode(const moe_attn_dims *dims, const uint16_t *q, const uint16_t *k,
                                  const uint16_t *v, uint16_t *o, void *ws, size_t ws_bytes, void *stream);

/* Measurement form of moe_gqa_decode: kernel i (0: splits, 1: combine) is
 * launched with events[2i] and events[2i+1] as its start and stop events;
 * needs n_events >= 4.  Not for use under stream capture. */
MOE_API moe_status moe_gqa_decode_timed(const moe_attn_dims *dims, const uint16_t *q, const uint16_t *k,
                                        const uint16_t *v, uint16_t *o, void *ws, size_t ws_bytes,
                                        void *stream, void *const *events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
