#!/usr/bin/env python3
"""Throughput of the MoE FFN layer on one MI355X, against its roofline.

One step = one pass of the whole layer (routing: top-k, histogram, scan,
scatter, block map; expert FFN: gate/up, SwiGLU, down, weighted combine with
the shared expert) over one batch of synthetic input already resident in HBM.

Primary line (`value`): batch-1 decode, T = 1 token per step, d = 2048,
E = 256, top-8 + shared, F = Fs = 512, int4 groups of 64, cycling through 40
distinct layer weight sets (455 MB each, 18.2 GB in all) so that weights
stream from HBM and not from cache; each step has its own x and logits.  The
K timed steps are one HIP graph of K layer calls.

Further objects: `prefill` (T = 4096 tokens with Zipf-skewed routing, the
prefill half of the metric), `prefill512` (T = 512) and `prefill32768`
(T = 32768), one weight set each, timed the same way; `attention`: the
second decode workload, attention of one token over grouped KV heads at
three cache lengths (context, not the metric).  The decode graph
visits min(K, 40) weight sets and the caches are flushed before every timed
replay, so the weights always come from HBM.

Per-kernel durations come from HIP start/stop events of each dispatch
(moe_layer_timed launches every kernel through hipExtLaunchKernel with an
event pair), taken on the same K steps run eagerly right after the timed
graph replay.  `cpu_baseline` times
the fp64 CPU oracle (test infrastructure) on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
METRIC = "MoE-layer tokens/s, prefill T=4096 & decode T=1; % of MFMA/HBM peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(kernel):
    """HBM bytes per dispatch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-kernel scaled), or None when there is none
    or the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            k = json.load(f)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    from bit_moe_expert_03_amd.profsum import source_hash
    if source_hash(k["sources"]) != k["source_sha256"]:
        return None
    return k["traffic_bytes"]


def achievable_peaks():
    """Context for the roofline fractions: what library code reaches on this
    box -- a device-to-device copy of 1 GiB (bytes read + written per
    second) and a 8192^3 bf16 matrix product on contiguous operands."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    for _ in range(3):
        dst.copy_(src)
        c = a @ b
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    for _ in range(10):
        c = a @ b
    e2.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / 10
    mm_s = e1.elapsed_time(e2) / 1e3 / 10
    out = {"hbm_copy_gbs": 2 * src.numel() * 4 / copy_s / 1e9, "bf16_matmul_tflops": 2 * 8192 ** 3 / mm_s / 1e12,
           "how": "torch copy_ of 1 GiB (read + write) and torch bf16 8192^3 matmul, 10 reps each"}
    del src, dst, a, b, c
    torch.cuda.empty_cache()
    return out


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs visible"


def copy_calibration(mb):
    """A plain copy kernel of known size (int32 x 1 into a second buffer),
    run three times so that counter passes can scale FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.ones((mb << 20) // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # materialise the underlying hipEvent_t
    torch.cuda.synchronize()
    return evs


def gateup_decode_bytes(dims):
    """Algorithmic bytes of the decode gate/up kernel: packed codes + bf16
    scale/bias of gate and up for the k routed and the shared expert, x,
    the logits row, and the bf16 h it writes."""
    per_row = dims.d // 2 + 2 * 2 * (dims.d // dims.G)
    w = 2 * per_row * (dims.k * dims.F + dims.Fs)
    return w + dims.d * 2 + dims.E * 4 + (dims.k * dims.F + dims.Fs) * 2


def decode_layer_bytes(dims):
    """Algorithmic bytes of one decode layer: weights of the k + 1 experts
    used (codes + scale/bias of gate, up, down), x and y."""
    gu = dims.d // 2 + 4 * (dims.d // dims.G)
    dn_r = dims.F // 2 + 4 * (dims.F // dims.G)
    dn_s = dims.Fs // 2 + 4 * (dims.Fs // dims.G)
    w = 2 * gu * (dims.k * dims.F + dims.Fs) + dims.d * (dims.k * dn_r + dn_s)
    return w + 2 * dims.d * 2


def gateup_flops(dims):
    """Useful matrix-core flops of the gate/up GEMM: 2 flops x 2 matrices x d
    for every (row, column) of the routed rows and the shared rows."""
    return 4 * dims.d * (dims.T * dims.k * dims.F + dims.T * dims.Fs)


def layer_flops(dims):
    return dims.T * (dims.k * 6 * dims.d * dims.F + 6 * dims.d * dims.Fs)


class CacheFlush:
    """Evicts the 256 MB Infinity Cache and the L2s between timed replays
    (outside the timed region): a device copy of 1 GiB."""

    def __init__(self):
        import torch
        self.src = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.dst.copy_(self.src)


def run_timed(B, dm, calls, steps, warmup, flush=None, queue_ahead=False):
    """calls[i] = (logits, x, weights_struct, y) for step i % len(calls).

    Timed region: one HIP graph of `steps` consecutive layer calls, replayed
    once untimed (upload) and three times timed between device
    synchronisations (median); with `flush`, the caches are flushed before
    each replay, outside the timed region.  Per-kernel times: right after,
    the same `steps` calls eagerly through moe_layer_timed, whose kernels are
    launched with start/stop events (hipExtLaunchKernel) on the launch
    stream (with `queue_ahead`, behind a spin kernel, so that they run back
    to back).  Returns (seconds, mean ms per kernel)."""
    import torch
    nk = B.moe_layer_kernels(dm)
    r = B.alloc_routing(dm)
    ws = B.alloc_workspace(dm)
    for i in range(warmup):
        lg, x, w, y = calls[i % len(calls)]
        B.moe_layer(dm, lg, x, w, r, y, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                lg, x, w, y = calls[i % len(calls)]
                B.moe_layer(dm, lg, x, w, r, y, ws, stream=stream)
    torch.cuda.synchronize()
    g.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):  # median of three timed replays
        if flush:
            flush()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        reps.append(time.perf_counter() - t0)
    reps.sort()
    evs = [make_events(2 * nk) for _ in range(steps)]
    if flush:
        flush()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        if queue_ahead:
            # a spin kernel first (about 0.1 s of shader clocks), so that the
            # eager launches queue up behind it and then run back to back as
            # in the graph, instead of one by one as the host submits them
            # (a decode layer's two kernels take less GPU time than the host
            # takes to submit them with their events)
            torch.cuda._sleep(200_000_000)
        for i in range(steps):
            lg, x, w, y = calls[i % len(calls)]
            B.moe_layer_timed(dm, lg, x, w, r, y, ws, [e.cuda_event for e in evs[i]], stream=stream)
    torch.cuda.synchronize()
    per_kernel = [sum(ev[2 * j].elapsed_time(ev[2 * j + 1]) for ev in evs) / steps for j in range(nk)]
    return reps[1], per_kernel


def bench_decode(B, wl, args):
    import torch
    name = "c1_decode"
    dims = wl.CONFIGS[name]
    seed = wl.SEED_OF[name]
    nsets = wl.DECODE_WEIGHT_SETS
    dm = B.make_dims(dims)
    sets, host_sets = [], []
    t = time.time()
    for s in range(nsets):
        W = wl.make_weights(dims, seed, s)
        wd = {m: {f: to_dev(W[m][f]) for f in ("q", "s", "b")} for m in wl.MATS}
        sets.append((wd, B.weights_struct(wd)))
        if s < 2:
            host_sets.append(W)
        if s % 10 == 9:
            log(f"decode: {s + 1}/{nsets} weight sets resident ({time.time() - t:.0f} s)")
    calls, host_inputs = [], []
    for s in range(nsets):
        c = wl.make_case(dims, seed=seed, index=s, weights=False)
        y = torch.empty((1, dims.d), dtype=torch.int16, device="cuda")
        calls.append((to_dev(c["logits"]), to_dev(c["x"]), sets[s][1], y))
        host_inputs.append(c)
    log("decode: capturing and timing")
    flush = CacheFlush()
    sec, per_kernel = run_timed(B, dm, calls, args.steps, args.warmup, flush, queue_ahead=True)
    value = args.steps / sec
    names, kernel = ["decode_gateup", "decode_down"], "decode_gateup_kernel"
    dom_bytes = gateup_decode_bytes(dims)
    dom_ms = per_kernel[0]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    out = {
        "value": value,
        "ms_per_step": sec * 1e3 / args.steps,
        "per_kernel_ms": dict(zip(names, per_kernel)),
        "layer_bytes": decode_layer_bytes(dims),
        "layer_gbs": decode_layer_bytes(dims) / (sec / args.steps) / 1e9,
        "weight_sets_touched_per_replay": min(args.steps, nsets),
        "bytes_touched_per_replay": min(args.steps, nsets) * decode_layer_bytes(dims),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(kernel), "bytes_per_launch": dom_bytes,
                     "avg_launch_ms": dom_ms},
    }
    log(f"decode: {value:.0f} tok/s, {out['ms_per_step'] * 1e3:.2f} us/step, "
        + ", ".join(f"{n} {t * 1e3:.2f} us" for n, t in zip(names, per_kernel)) + f" ({achieved:.0f} GB/s)")
    del flush
    out["small_batches"] = None if args.no_small_batches else bench_small_batches(B, wl, args, dims, seed, sets)
    del sets, calls
    torch.cuda.empty_cache()
    return out, (dims, host_sets, host_inputs)


def bench_small_batches(B, wl, args, dims, seed, sets):
    """Context, not the metric: few-token batches (the verify passes of
    speculative decoding) at the decode layer shape over the same rotated
    weight sets, one graph of args.steps // 4 layer calls per batch size."""
    import torch
    out = {}
    steps = max(8, args.steps // 4)
    for T in (2, 4, 8, 16, 32):
        dT = dims.replace(T=T)
        dm = B.make_dims(dT)
        calls = []
        for s in range(len(sets)):
            c = wl.make_case(dT, seed=seed, index=1000 + 40 * T + s, weights=False)
            y = torch.empty((T, dims.d), dtype=torch.int16, device="cuda")
            calls.append((to_dev(c["logits"]), to_dev(c["x"]), sets[s][1], y))
        sec, per_kernel = run_timed(B, dm, calls, steps, 8, queue_ahead=True)
        out[f"T{T}"] = {"tokens_per_s": T * steps / sec, "us_per_step": sec * 1e6 / steps,
                        "per_kernel_us": [k * 1e3 for k in per_kernel]}
        log(f"small batch T={T}: {sec * 1e6 / steps:.1f} us/step, {T * steps / sec:.0f} tok/s")
    return out


PREFILL_WORKLOADS = {
    # key in the JSON line: (workload name, description)
    "prefill": ("c3_prefill4096_zipf", "prefill T=4096 Zipf(1)-skewed routing"),
    "prefill512": ("c2_prefill512", "prefill T=512 near-uniform routing"),
    "prefill32768": ("c4_prefill32768", "prefill T=32768 near-uniform routing"),
}


def bench_prefill(B, wl, args, name, desc, steps):
    """One prefill workload: the whole layer (routing + FFN) from device
    logits and x to device y, one weight set, `steps` layer calls in a graph;
    roofline of the gate/up GEMM (useful bf16 MFMA flops per launch)."""
    import torch
    c = wl.make_case(name)
    dims = c["dims"]
    dm = B.make_dims(dims)
    wd = {m: {f: to_dev(c["w"][m][f]) for f in ("q", "s", "b")} for m in wl.MATS}
    y = torch.empty((dims.T, dims.d), dtype=torch.int16, device="cuda")
    calls = [(to_dev(c["logits"]), to_dev(c["x"]), B.weights_struct(wd), y)]
    log(f"{name}: capturing and timing")
    sec, per_kernel = run_timed(B, dm, calls, steps, 3)
    names = ["route_topk", "route_scan", "route_scatter", "gateup_gemm", "down_gemm", "combine"]
    value = dims.T * steps / sec
    gu_ms = per_kernel[3]
    fl = gateup_flops(dims)
    achieved = fl / (gu_ms * 1e-3) / 1e12
    ms = sec * 1e3 / steps
    out = {
        "value": value, "unit": "tokens/s", "ms_per_step": ms, "steps": steps,
        "dtype": "bf16",
        "config": {"workload": f"{desc}, d=2048, E=256, top-8 + shared, F=Fs=512, int4 G=64, one weight set",
                   "T": dims.T},
        "per_kernel_ms": dict(zip(names, per_kernel)),
        "routing_gbs": (dims.T * dims.E * 4 + dims.T * dims.k * 16) / (sum(per_kernel[:3]) * 1e-3) / 1e9,
        "layer_tflops": layer_flops(dims) / (ms * 1e-3) / 1e12,
        "layer_mfma_frac": layer_flops(dims) / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "roofline": {"bound": "mfma", "kernel": "moe_gateup_kernel", "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFS,
                     "traffic": measured_traffic("moe_gateup_kernel") if name == "c3_prefill4096_zipf" else None,
                     "flops_per_launch": fl, "avg_launch_ms": gu_ms},
    }
    log(f"{name}: {value / 1e6:.2f} M tok/s, {ms * 1e3:.1f} us/step, kernels "
        + ", ".join(f"{n} {t * 1e3:.1f}us" for n, t in zip(names, per_kernel)))
    if name == "c3_prefill4096_zipf":
        out["route_from_x"] = bench_route_x(B, wl, c, dm)
    del wd, calls, y
    torch.cuda.empty_cache()
    return out, c


def bench_route_x(B, wl, c, dm, reps=20):
    """Context: routing from the activations (router projection on the GPU,
    then the routing kernels) against routing from given logits, per call."""
    import torch
    dims = c["dims"]
    wr = wl.make_router(dims, c["seed"])
    bias = wl.zipf_bias(dims.E, c["seed"]).astype("float32")
    packed = torch.empty(B.moe_router_packed_bytes(dm) // 2, dtype=torch.int16, device="cuda")
    B.moe_router_pack(dm, to_dev(wr), packed)
    x, bd, lg_in = to_dev(c["x"]), to_dev(bias), to_dev(c["logits"])
    lg = torch.empty((dims.T, dims.E), dtype=torch.float32, device="cuda")
    r = B.alloc_routing(dm)
    ws = B.alloc_workspace(dm)
    res = {}
    for label, f in (("route_x_us", lambda: B.moe_route_x(dm, x, packed, bd, lg, r, ws)),
                     ("route_us", lambda: B.moe_route(dm, lg_in, r, ws))):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        res[label] = e0.elapsed_time(e1) / reps * 1e3
    res["router_tflops"] = 2.0 * 2 * dims.T * dims.d * dims.E / ((res["route_x_us"] - res["route_us"]) * 1e-6) / 1e12
    log(f"prefill: routing from x {res['route_x_us']:.1f} us/call (from logits {res['route_us']:.1f})")
    return res


def attn_bytes(a):
    """Algorithmic bytes of one decode-attention call: the K and V caches of
    every KV head, q read and o written (bf16); the kernels' fp32 partials
    are the implementation's, not the algorithm's."""
    return 2 * a.Hkv * a.L * a.D * 2 + 2 * a.Hq * a.D * 2


def bench_attn(B, wl, args, name, calls=200):
    """Context, the second decode workload: attention of one token over a
    KV cache of L tokens, eight query heads per KV head.  Distinct KV caches
    (the layers of a model) rotate per call, about 2 GiB in all, so every
    call streams its cache from HBM.  Timed: one HIP graph of `calls` calls
    (median of three replays); per-kernel times from event pairs on the
    same calls run eagerly behind a spin kernel."""
    import torch
    a = wl.ATTN_CONFIGS[name]
    ad = B.make_attn_dims(a)
    per = attn_bytes(a)
    nsets = max(2, min(calls, -(-(2 << 30) // per)))
    c = wl.make_attn_case(name)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    sets = [(to_dev(c["k"]), to_dev(c["v"]))]
    for _ in range(nsets - 1):
        kv = torch.randn((2, a.Hkv, a.L, a.D), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
        sets.append((kv[0], kv[1]))
    q = to_dev(c["q"])
    o = torch.empty((a.Hq, a.D), dtype=torch.int16, device="cuda")
    ws = B.alloc_gqa_workspace(ad)
    for i in range(3):
        B.moe_gqa_decode(ad, q, sets[i % nsets][0], sets[i % nsets][1], o, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(calls):
                B.moe_gqa_decode(ad, q, sets[i % nsets][0], sets[i % nsets][1], o, ws, stream=stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        reps.append(time.perf_counter() - t0)
    sec = sorted(reps)[1] / calls
    evs = [make_events(4) for _ in range(calls)]
    with torch.cuda.stream(stream):
        torch.cuda._sleep(200_000_000)
        for i in range(calls):
            B.moe_gqa_decode_timed(ad, q, sets[i % nsets][0], sets[i % nsets][1], o, ws,
                                   [e.cuda_event for e in evs[i]], stream=stream)
    torch.cuda.synchronize()
    per_kernel = [sum(ev[2 * j].elapsed_time(ev[2 * j + 1]) for ev in evs) / calls for j in range(2)]
    achieved = per / (per_kernel[0] * 1e-3) / 1e9
    out = {
        "workload": f"decode attention, one token over L={a.L} cached tokens, Hq={a.Hq} query heads on "
                    f"Hkv={a.Hkv} KV heads (8 per KV head), D={a.D}, bf16 K/V cache, {nsets} caches rotated",
        "us_per_call": sec * 1e6,
        "calls_per_s": 1.0 / sec,
        "gbs_per_call": per / sec / 1e9,
        "bytes_per_call": per,
        "per_kernel_us": {"gqa_partial": per_kernel[0] * 1e3, "gqa_combine": per_kernel[1] * 1e3},
        "roofline": {"bound": "hbm", "kernel": "gqa_partial_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("gqa_partial_kernel_" + name.split("_")[-1]),
                     "bytes_per_launch": per, "avg_launch_ms": per_kernel[0]},
    }
    log(f"attention {name}: {sec * 1e6:.2f} us/call ({out['gbs_per_call']:.0f} GB/s), partial "
        f"{per_kernel[0] * 1e3:.2f} us ({achieved:.0f} GB/s), combine {per_kernel[1] * 1e3:.2f} us")
    if not args.no_cpu_baseline:
        import oracle
        t0, n = time.perf_counter(), 0
        while True:
            oracle.gqa_decode(c["q"], c["k"], c["v"])
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds / 4:
                break
        out["cpu_baseline"] = {"value": n / el, "unit": "calls/s", "cores": oracle.threads(), "kind": "oracle",
                               "sample": f"{n} fp64 oracle calls on the first cache of this workload "
                                         "(OpenMP over query heads)"}
    del sets, g
    torch.cuda.empty_cache()
    return out


def cpu_baseline_decode(wl, host, seconds):
    """The oracle on decode tokens: each call routes and runs the fp64 FFN of
    a batch of independent T = 1 decode steps that share one weight set, so
    the oracle's OpenMP loop over tokens uses every host core."""
    import numpy as np
    import oracle
    dims, host_sets, host_inputs = host
    nb = max(1, oracle.threads())
    t0 = time.perf_counter()
    n, calls = 0, 0
    while True:
        cs = [host_inputs[(n + i) % len(host_inputs)] for i in range(nb)]
        x = np.concatenate([c["x"] for c in cs])
        lg = np.concatenate([c["logits"] for c in cs])
        r = oracle.route(lg, dims.k, 32)
        oracle.ffn(dims.replace(T=nb), x, host_sets[calls % len(host_sets)], r["ids"], r["w"])
        n += nb
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n / el, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle", "host": host_cpu(),
            "sample": f"{n} decode tokens (T=1 steps: route + fp64 FFN), {nb} independent steps per oracle call "
                      f"sharing one of {len(host_sets)} weight sets, OpenMP over the steps"}


def cpu_baseline_prefill(wl, c, seconds):
    import oracle
    dims = c["dims"]
    t0 = time.perf_counter()
    r = oracle.route(c["logits"], dims.k, 128)
    ntok, n = 0, 64
    while True:
        toks = list(range(ntok, ntok + n))
        oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=toks)
        ntok += n
        el = time.perf_counter() - t0
        if el >= seconds or ntok + n > dims.T:
            break
    return {"value": ntok / el, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle", "host": host_cpu(),
            "sample": f"routing of all {dims.T} tokens + fp64 FFN of the first {ntok} tokens of the "
                      f"T={dims.T} workload (OpenMP over tokens)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=40, help="untimed decode steps")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-small-batches", action="store_true",
                    help="skip the few-token batch context (counter passes keep the decode kernels at T=1)")
    ap.add_argument("--no-attn", action="store_true", help="skip the decode-attention context")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="first run a plain copy kernel of this many MB (scale for counter passes)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_moe_expert_03_amd import binding as B
    from bit_moe_expert_03_amd import workload as wl
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()  # fails loudly if the HIP library is not built
    if args.copy_calib_mb:
        copy_calibration(args.copy_calib_mb)

    peaks = achievable_peaks()
    log(f"achievable: copy {peaks['hbm_copy_gbs']:.0f} GB/s, bf16 matmul {peaks['bf16_matmul_tflops']:.0f} TFLOP/s")
    dec, host = bench_decode(B, wl, args)
    dec["roofline"]["frac_of_achievable"] = dec["roofline"]["achieved"] / peaks["hbm_copy_gbs"]
    pre = {}
    if not args.no_prefill:
        for key, (name, desc) in PREFILL_WORKLOADS.items():
            steps = args.prefill_steps if name != "c4_prefill32768" else max(3, args.prefill_steps // 4)
            out, case = bench_prefill(B, wl, args, name, desc, steps)
            out["roofline"]["frac_of_achievable"] = out["roofline"]["achieved"] / peaks["bf16_matmul_tflops"]
            if not args.no_cpu_baseline:
                out["cpu_baseline"] = cpu_baseline_prefill(wl, case, args.cpu_seconds)
            pre[key] = out
            del case
    attn = None
    if not args.no_attn:
        attn = {name: bench_attn(B, wl, args, name) for name in wl.ATTN_CONFIGS}
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline_decode(wl, host, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": dec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "int4 groupwise-affine weights, bf16 activations and products, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": "decode T=1, d=2048, E=256, top-8 + shared, F=Fs=512, int4 G=64, "
                               "40 layer weight sets rotated per step, caches flushed before each timed replay",
                   "T": 1, "weight_sets": 40, "weight_sets_touched_per_replay": min(args.steps, 40)},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_detail": {k: dec[k] for k in ("per_kernel_ms", "layer_bytes", "layer_gbs", "small_batches")},
        "prefill": pre.get("prefill"),
        "prefill512": pre.get("prefill512"),
        "prefill32768": pre.get("prefill32768"),
        "attention": attn,
        "achievable": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
