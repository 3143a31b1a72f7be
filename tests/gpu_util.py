"""Helpers of the GPU parity tests: upload seeded inputs, run the C ABI through
the binding, bring results back, compare with the oracle.

Every output array and the workspace are allocated with a guard band of 256
bytes on each side, filled with a canary pattern; after each call the bands
must still hold it, so a write past either end of any array fails the test
(the outputs themselves are pre-filled with a NaN / -7 poison pattern, so an
element the kernels fail to write fails as well).  Each y comparison records
max|y - y_ref| / tolerance; with PARITY_LOG set, one JSON line per comparison
is appended to that file."""
import json
import os

import numpy as np
import torch

import oracle
from bit_moe_expert_03_amd import binding as B
from bit_moe_expert_03_amd import workload as wl

GUARD_BYTES = 256
CANARY_BYTE = 0x5A


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def weights_to_dev(W):
    return {m: {f: dev(W[m][f]) for f in ("q", "s", "b")} for m in wl.MATS}


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Guarded:
    """A device array with canary bands of GUARD_BYTES before and after it.
    `t` is the payload (16-byte aligned, contiguous); `check()` raises if a
    band changed."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(shape)
        n = int(np.prod(shape)) if shape else 1
        esize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = n * esize
        self.buf = torch.full((2 * GUARD_BYTES + self.nbytes,), CANARY_BYTE, dtype=torch.uint8, device="cuda")
        payload = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes]
        self.t = payload.view(dtype).view(shape) if n else torch.empty(shape, dtype=dtype, device="cuda")
        if fill is not None and n:
            self.t.fill_(fill)

    def check(self, what):
        b = self.buf.cpu().numpy()
        front, back = b[:GUARD_BYTES], b[GUARD_BYTES + self.nbytes:]
        assert np.all(front == CANARY_BYTE), f"{what}: write before the start of the array"
        assert np.all(back == CANARY_BYTE), f"{what}: write past the end of the array"


def guarded_routing(dm, poison=True):
    """Routing outputs (as binding.alloc_routing) inside guard bands."""
    A = dm.T * dm.k
    mt = B.moe_max_tiles(dm)
    shapes = {"topk_ids": ((dm.T, dm.k), torch.int32), "topk_w": ((dm.T, dm.k), torch.float32),
              "counts": ((dm.E,), torch.int32), "offsets": ((dm.E + 1,), torch.int32),
              "perm": ((A,), torch.int32), "inv_perm": ((A,), torch.int32),
              "tile_expert": ((mt,), torch.int32), "tile_row0": ((mt,), torch.int32),
              "tile_rows": ((mt,), torch.int32), "num_tiles": ((1,), torch.int32)}
    g = {}
    for name, (shape, dt) in shapes.items():
        g[name] = Guarded(shape, dt)
        if poison and g[name].t.numel():
            if dt == torch.float32:
                g[name].t.view(torch.int32).fill_(-7)
            else:
                g[name].t.fill_(-7)
    return g


def guarded_workspace(dm):
    """Workspace in guard bands; zero-filled before its first use, as the
    ABI asks."""
    n = max(B.moe_workspace_bytes(dm), 256)
    return Guarded((n,), torch.uint8, fill=0)


def run(case, tile_m=0, mode="layer", wdev=None, poison=True, down_nc=0):
    """Run the layer on the GPU.  mode: 'layer' (moe_layer), 'split'
    (moe_route then moe_ffn).  Returns host copies of every output; every
    guard band is checked."""
    dims = case["dims"]
    dm = B.make_dims(dims, tile_m, down_nc=down_nc)
    wdev = wdev if wdev is not None else weights_to_dev(case["w"])
    if case.get("shared_gate") is not None:
        wdev = dict(wdev, shared_gate=dev(case["shared_gate"]))
    logits = dev(case["logits"])
    x = dev(case["x"])
    gr = guarded_routing(dm, poison)
    r = {k: v.t for k, v in gr.items()}
    gws = guarded_workspace(dm)
    gy = Guarded((dims.T, dims.d), torch.int16, fill=0x7FC1 if poison else 0)  # NaN pattern
    if mode == "layer":
        B.moe_layer(dm, logits, x, wdev, r, gy.t, gws.t)
    else:
        B.moe_route(dm, logits, r, gws.t)
        B.moe_ffn(dm, x, wdev, r, gy.t, gws.t)
    torch.cuda.synchronize()
    for k, v in gr.items():
        v.check(k)
    gws.check("workspace")
    gy.check("y")
    out = {k: v.cpu().numpy() for k, v in r.items()}
    out["y_bits"] = host_u16(gy.t)
    out["y"] = bf16_to_f64(out["y_bits"])
    out["tile_m"] = B.moe_tile_m(dm)
    out["max_tiles"] = B.moe_max_tiles(dm)
    return out


def check_routing(case, g):
    """Routing outputs bit-exact against the oracle; weights within 1e-6."""
    dims = case["dims"]
    ref = oracle.route(case["logits"], dims.k, g["tile_m"], g["max_tiles"])
    np.testing.assert_array_equal(g["topk_ids"], ref["ids"])
    np.testing.assert_array_equal(g["counts"], ref["counts"])
    np.testing.assert_array_equal(g["offsets"], ref["offsets"])
    np.testing.assert_array_equal(g["perm"], ref["perm"])
    np.testing.assert_array_equal(g["inv_perm"], ref["inv_perm"])
    n = int(g["num_tiles"][0])
    assert n == ref["num_tiles"]
    np.testing.assert_array_equal(g["tile_expert"][:n], ref["tile_expert"])
    np.testing.assert_array_equal(g["tile_row0"][:n], ref["tile_row0"])
    np.testing.assert_array_equal(g["tile_rows"][:n], ref["tile_rows"])
    if dims.T:
        assert np.abs(g["topk_w"].astype(np.float64) - ref["w"]).max() <= 1e-6
        assert np.abs(g["topk_w"].astype(np.float64).sum(1) - 1.0).max() <= 1e-6
    return ref


def y_tolerance(y_ref: np.ndarray) -> float:
    """max|y - y_ref| <= 1e-2 max|y_ref| + 1e-3 (bf16 outputs vs fp64 oracle)."""
    return 1e-2 * float(np.abs(y_ref).max()) + 1e-3


_YREF = {}


def oracle_y(case, ref_route, tokens=None, key=None):
    """The oracle's y for all tokens or the listed ones; memoised under `key`
    (the same workload compared in several tests)."""
    ck = None if key is None else (key, None if tokens is None else tuple(int(t) for t in tokens))
    if ck is not None and ck in _YREF:
        return _YREF[ck]
    dims = case["dims"]
    y_ref = oracle.ffn(dims, case["x"], case["w"], ref_route["ids"], ref_route["w"], tokens=tokens,
                       shared_gate=case.get("shared_gate"))
    if ck is not None:
        _YREF[ck] = y_ref
    return y_ref


def log_margin(label, err, tol, ntok, T):
    line = {"case": label, "err": err, "tol": tol, "err_over_tol": err / tol, "tokens": ntok, "T": T}
    print(f"[parity] {label}: max err {err:.4g} / tol {tol:.4g} = {err / tol:.3f} over {ntok} of {T} tokens",
          flush=True)
    path = os.environ.get("PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def check_y(case, g, ref_route, tokens=None, key=None, label=None):
    """y against the oracle on all tokens, or on the listed ones."""
    dims = case["dims"]
    y_ref = oracle_y(case, ref_route, tokens, key)
    y = g["y"] if tokens is None else g["y"][np.asarray(tokens, dtype=np.int64)]
    assert np.all(np.isfinite(g["y"])), "unwritten or non-finite outputs"
    err = float(np.abs(y - y_ref).max()) if y.size else 0.0
    tol = y_tolerance(y_ref) if y.size else 1.0
    log_margin(label or key or str(dims), err, tol, dims.T if tokens is None else len(tokens), dims.T)
    assert err <= tol, f"max|y - y_ref| = {err} > {tol}"
    return err, tol


def tile_tokens(case, ref_route, tile_m):
    """Tokens that put a row into every tile the GEMM kernels run: the first
    and last sorted row of every routed block-map tile (through perm), the
    first and last token of every shared-expert tile (tile_m consecutive
    tokens), and the first and last few tokens."""
    T, k = case["dims"].T, case["dims"].k
    perm = ref_route["perm"]
    row0 = np.asarray(ref_route["tile_row0"], np.int64)
    rows = np.asarray(ref_route["tile_rows"], np.int64)
    pick = set((perm[row0] // k).tolist()) | set((perm[row0 + rows - 1] // k).tolist())
    starts = np.arange(0, T, tile_m)
    pick |= set(starts.tolist()) | set(np.minimum(starts + tile_m - 1, T - 1).tolist())
    pick |= set(range(min(4, T))) | set(range(max(0, T - 4), T))
    return sorted(int(t) for t in pick)
