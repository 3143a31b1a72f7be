// Batch-1 decode path of the MoE layer (gfx950): matrix-vector kernels that
// stream the packed 4-bit weights of the k routed experts and the shared
// expert at HBM rate, with wave reductions and no matrix cores.  The Lily
// pages run batch-1 decode on the vector ALUs because one token gives no
// weight reuse, so the pass is bound by memory bandwidth (page "Perplexity's
// Lily Beats MLX-LM by 1.35x Running Qwen3.6 on Apple Silicon", section "Why
// prefill and decode get different treatment").
//
// The same two kernels serve batches of up to kMaxDecodeT tokens (the
// pages' few-token verify passes): every work wave and down block belongs to
// one token, and an expert chosen by several tokens is streamed once per
// token (the repeats mostly hit L2 / Infinity Cache).
//
// Two kernels per layer:
//   decode_gateup_kernel  block 0: top-k + softmax of every token's logits
//                         and the routing outputs (sorted order, counts,
//                         offsets, block map), and the shared expert's gate
//                         values when it is gated.  Every other wave owns
//                         P (gate, up) row pairs of one expert slot
//                         and writes h_j[n] = bf16(silu(W_gate,j[n] . x) *
//                         (W_up,j[n] . x)).  A wave of routed slot j needs
//                         only the expert of rank j, so it runs the top-k
//                         rounds 0..j itself (no block barrier) and issues
//                         its loads as soon as that expert is known; the
//                         shared expert's waves load at once.  Slots are
//                         ordered k-1 .. 0, shared last, so the waves with
//                         the longest top-k are dispatched first.
//   decode_down_kernel    y[i] = sum_j w_j (W_down,j[i] . h_j) + gamma W_sdown[i] . h_s,
//                         kDownRows output rows per block; lane = one
//                         32-element chunk of the concatenated hidden vector
//                         (shared expert first, its loads need no routing).
//
// The 4-bit dot products (factored affine form, v_dot2_f32_bf16) are in
// decode_common.h.
#include "decode_common.h"

namespace moe {

constexpr int kDecThreads = 256;  // 4 waves per block
constexpr int kDownRows = 2;      // output rows per down block
constexpr int kDownMaxThreads = 512;
constexpr int kMaxDecodeA = kMaxDecodeAssign;  // assignments of a batch

struct DecodeArgs {
    const float *logits;  // [T][E] or null (routing given in r)
    const uint16_t *x;    // [T][d]
    moe_weights w;
    moe_routing r;
    int T, d, E, k, F, Fs, G, Fmax, tile_m;
    int wps_r, wps_s;     // work waves per routed slot, for the shared expert
    uint16_t *h;          // [T][k+1][Fmax] bf16 workspace: slots 0..k-1 routed, k shared
    float *gamma;         // [T] workspace: weight of the shared expert (gated variant)
    uint16_t *y;          // [T][d]
};

// ---- routing -----------------------------------------------------------------

// block 0 of the gate/up grid: top-k, softmax over the k chosen logits of
// each token (wave w takes tokens w, w + 4, ...)
__device__ void decode_routing_block(const DecodeArgs &a)
{
    __shared__ int s_ids[kMaxDecodeA];
    __shared__ float s_w[kMaxDecodeA];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int t = wave; t < a.T; t += kDecThreads / kWave) {
        TopK tk;
        wave_topk(load_logits(a.logits + (size_t)t * a.E, a.E), a.E, a.k, tk);
        float ex[4], part = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = lane + 64 * c;
            ex[c] = (j < a.k) ? expf(tk.logit[c] - tk.lmax) : 0.f;
            part += ex[c];
        }
        const float inv = 1.0f / wave_sum(part);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = lane + 64 * c;
            if (j < a.k) { s_ids[t * a.k + j] = tk.id[c]; s_w[t * a.k + j] = ex[c] * inv; }
        }
    }
    __syncthreads();
    decode_write_routing(a.r, a.T, a.E, a.k, s_ids, s_w);
}

// block 0 of the gate/up grid, gated shared expert: gamma_t = sigmoid(x_t . g)
__device__ void decode_shared_gate(const DecodeArgs &a)
{
    __shared__ float part[kDecThreads / kWave];
    const int tid = threadIdx.x;
    for (int t = 0; t < a.T; ++t) {
        const uint16_t *xt = a.x + (size_t)t * a.d;
        float z = 0.f;
        for (int c = tid * 8; c < a.d; c += kDecThreads * 8) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xt + c);
            const uint4 gv = *reinterpret_cast<const uint4 *>(a.w.shared_gate + c);
            z = dot2_bf16(xv.x, gv.x, z);
            z = dot2_bf16(xv.y, gv.y, z);
            z = dot2_bf16(xv.z, gv.z, z);
            z = dot2_bf16(xv.w, gv.w, z);
        }
        z = wave_sum(z);
        if ((tid & 63) == 0) part[tid >> 6] = z;
        __syncthreads();
        if (tid == 0) {
            float v = 0.f;
            for (int w = 0; w < kDecThreads / kWave; ++w) v += part[w];
            a.gamma[t] = 1.0f / (1.0f + __expf(-v));
        }
        __syncthreads();
    }
}

// ---- gate/up -------------------------------------------------------------------

// NCH = 32-element chunks of x per lane (d <= 2048 * NCH); P row pairs per wave
template <int NCH, int P>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs a)
{
    if (blockIdx.x == 0) {
        if (a.logits) decode_routing_block(a);
        if (a.w.shared_gate) decode_shared_gate(a);
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per_token = a.k * a.wps_r + a.wps_s;  // work waves of one token
    const int gw0 = (blockIdx.x - 1) * (kDecThreads / kWave) + wave;
    const int t = gw0 / per_token;
    if (t >= a.T) return;
    const int gw = gw0 - t * per_token;  // work wave inside the token
    const int nchunk = a.d >> 5;
    int slot, n0;
    if (gw < a.k * a.wps_r) {
        slot = a.k - 1 - gw / a.wps_r;
        n0 = (gw % a.wps_r) * P;
    } else {
        slot = a.k;
        n0 = (gw - a.k * a.wps_r) * P;
    }
    const bool shared = slot == a.k;
    const uint16_t *xt = a.x + (size_t)t * a.d;

    // this lane's chunks of x: chunk c = lane + 64 i covers x[32c, 32c+32)
    uint4 xr[NCH][4];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < nchunk) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(xt + (size_t)c * 32);
#pragma unroll
            for (int v = 0; v < 4; ++v) xr[i][v] = xp[v];
        }
    }
    RowRaw rg[P][NCH], ru[P][NCH];
    const moe_qmat &mg = shared ? a.w.sgate : a.w.gate;
    const moe_qmat &mu = shared ? a.w.sup : a.w.up;
    size_t row0;
    if (shared) {
        row0 = (size_t)n0;
    } else {
        int e;
        if (a.logits) {
            // the four waves of a block share the token and the slot (the
            // waves of a token and of a slot are multiples of four): wave 0
            // runs the selection rounds and hands the expert over through
            // LDS.  Rounds run by every wave keep the compute unit's scalar
            // unit busy and delay all of them (measured).
            __shared__ int s_expert;
            if (wave == 0) {
                uint32_t key[4];
                const LogitQuad lq = load_logits(a.logits + (size_t)t * a.E, a.E);
#pragma unroll
                for (int c = 0; c < 4; ++c) key[c] = (4 * lane + c < a.E) ? logit_key(lq.v[c]) : 0u;
                const int ew = wave_rank_expert(key, slot);
                if (lane == 0) s_expert = ew;
            }
            __syncthreads();
            e = s_expert;
        } else {
            e = min((uint32_t)a.r.topk_ids[t * a.k + slot], (uint32_t)(a.E - 1));  // ids from the caller: kept in range
        }
        row0 = (size_t)e * a.F + n0;
    }
#pragma unroll
    for (int pi = 0; pi < P; ++pi)
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + 64 * i;
            if (c < nchunk) {
                load_row(rg[pi][i], mg, row0 + pi, c, a.d, a.G);
                load_row(ru[pi][i], mu, row0 + pi, c, a.d, a.G);
            }
        }
    float accg[P], accu[P];
#pragma unroll
    for (int pi = 0; pi < P; ++pi) { accg[pi] = 0.f; accu[pi] = 0.f; }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c >= nchunk) continue;
        VecChunk xv;
        vec_chunk(xr[i], xv);
        uint4 q[2 * P];
        float dq[2 * P];
#pragma unroll
        for (int pi = 0; pi < P; ++pi) { q[2 * pi] = rg[pi][i].q; q[2 * pi + 1] = ru[pi][i].q; }
        dot_codes32_rows<2 * P>(q, xv, dq);
#pragma unroll
        for (int pi = 0; pi < P; ++pi) {
            accg[pi] += chunk_term(dq[2 * pi], xv, rg[pi][i].s, rg[pi][i].b);
            accu[pi] += chunk_term(dq[2 * pi + 1], xv, ru[pi][i].s, ru[pi][i].b);
        }
    }
    uint16_t *hrow = a.h + ((size_t)t * (a.k + 1) + slot) * a.Fmax + n0;
#pragma unroll
    for (int pi = 0; pi < P; ++pi) {
        const float g = wave_sum(accg[pi]);
        const float u = wave_sum(accu[pi]);
        if (lane == 0) hrow[pi] = f32_to_bf16(silu(g) * u);
    }
}

// ---- down ---------------------------------------------------------------------

// One block = kDownRows output rows of token blockIdx.y; lane chunks
// c = tid, tid + blockDim, ... of [h_s, h_0 .. h_{k-1}] in 32-element chunks.
// Row blocks are spread over the XCDs in contiguous ranges, so that the
// blocks reading one 128-byte line of scales or biases (8 rows) share an L2.
__global__ __launch_bounds__(kDownMaxThreads) void decode_down_kernel(DecodeArgs a)
{
    __shared__ float red[kDownMaxThreads / kWave][kDownRows];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nw = blockDim.x >> 6;
    const int rb = xcd_logical_block(blockIdx.x, (a.d + kDownRows - 1) / kDownRows);
    if (rb < 0) return;  // grid padding (block-uniform)
    const int row0 = rb * kDownRows;
    const int t = blockIdx.y;
    const int cF = a.F >> 5, cFs = a.Fs >> 5;
    const int nchunks = a.k * cF + cFs;
    float acc[kDownRows];
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) acc[r] = 0.f;
    for (int c = tid; c < nchunks; c += blockDim.x) {
        int j, f0, Fw;
        const moe_qmat *m;
        size_t ebase;
        float wj;
        if (c < cFs) {  // shared expert: no routing needed
            j = a.k; f0 = c * 32; Fw = a.Fs; m = &a.w.sdown;
            ebase = 0;
            wj = a.w.shared_gate ? a.gamma[t] : 1.0f;
        } else {
            j = (c - cFs) / cF; f0 = (c - cFs - j * cF) * 32; Fw = a.F; m = &a.w.down;
            ebase = (size_t)min((uint32_t)a.r.topk_ids[t * a.k + j], (uint32_t)(a.E - 1)) * a.d;
            wj = a.r.topk_w[t * a.k + j];
        }
        uint4 q[kDownRows];
        uint16_t s[kDownRows], b[kDownRows];
        const int grp = f0 / a.G;
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) {
            const size_t row = ebase + min(row0 + r, a.d - 1);
            q[r] = *reinterpret_cast<const uint4 *>(m->q + row * (size_t)(Fw >> 1) + (f0 >> 1));
            const size_t gi = row * (size_t)(Fw / a.G) + grp;
            s[r] = m->s[gi];
            b[r] = m->b[gi];
        }
        uint4 hr[4];
        const uint4 *hp = reinterpret_cast<const uint4 *>(a.h + ((size_t)t * (a.k + 1) + j) * a.Fmax + f0);
#pragma unroll
        for (int v = 0; v < 4; ++v) hr[v] = hp[v];
        VecChunk hv;
        vec_chunk(hr, hv);
        float dq[kDownRows];
        dot_codes32_rows<kDownRows>(q, hv, dq);
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) acc[r] += wj * chunk_term(dq[r], hv, s[r], b[r]);
    }
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == 0) red[wave][r] = v;
    }
    __syncthreads();
    if (tid < kDownRows && row0 + tid < a.d) {
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += red[w][tid];
        a.y[(size_t)t * a.d + row0 + tid] = f32_to_bf16(v);
    }
}

template <int NCH, int P>
static void launch_gateup(EventTrace *tr, DecodeArgs &a, hipStream_t s)
{
    a.wps_r = a.F / P;
    a.wps_s = a.Fs / P;
    // the selection hand-over above needs every block inside one slot of one token
    static_assert(kDecThreads / kWave == 4 && 64 % (4 * P) == 0, "F / P and Fs / P multiples of the block's 4 waves");
    const int waves = a.T * (a.k * a.wps_r + a.wps_s);
    const int nb = 1 + (waves + kDecThreads / kWave - 1) / (kDecThreads / kWave);
    launch(tr, decode_gateup_kernel<NCH, P>, dim3(nb), dim3(kDecThreads), 0, s, a);
}

hipError_t launch_decode(const Plan &p, const float *logits, const uint16_t *x,
                         const moe_weights &w, const moe_routing &r, uint16_t *y, void *ws,
                         hipStream_t s, EventTrace *tr)
{
    DecodeArgs a;
    a.logits = logits;
    a.x = x;
    a.w = w;
    a.r = r;
    a.T = p.T; a.d = p.d; a.E = p.E; a.k = p.k; a.F = p.F; a.Fs = p.Fs; a.G = p.G; a.tile_m = p.tile_m;
    a.Fmax = p.F > p.Fs ? p.F : p.Fs;
    a.h = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + p.off_dech);
    a.gamma = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_gamma);
    a.y = y;
    // F and Fs are multiples of 64, so every P below divides both
    const int nch = (p.d / 32 + kWave - 1) / kWave;
    if (nch <= 1)
        launch_gateup<1, 2>(tr, a, s);
    else if (nch <= 2)
        launch_gateup<2, 2>(tr, a, s);
    else if (nch <= 4)
        launch_gateup<4, 2>(tr, a, s);
    else
        launch_gateup<8, 1>(tr, a, s);
    const int nchunks = p.k * (p.F >> 5) + (p.Fs >> 5);
    int nw = (nchunks + kWave - 1) / kWave;
    nw = nw < 1 ? 1 : (nw > kDownMaxThreads / kWave ? kDownMaxThreads / kWave : nw);
    const int nb2 = ((p.d + kDownRows - 1) / kDownRows + 7) & ~7;  // a multiple of 8 (XCD ranges)
    launch(tr, decode_down_kernel, dim3(nb2, p.T), dim3(nw * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
