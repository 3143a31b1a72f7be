"""Helpers of the GPU parity tests: upload seeded inputs, run the C ABI through
the binding, bring results back, compare with the oracle."""
import numpy as np
import torch

import oracle
from bit_moe_expert_03_amd import binding as B
from bit_moe_expert_03_amd import workload as wl


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


def run(case, tile_m=0, mode="layer", wdev=None, poison=True):
    """Run the layer on the GPU.  mode: 'layer' (moe_layer), 'split'
    (moe_route then moe_ffn).  Returns host copies of every output."""
    dims = case["dims"]
    dm = B.make_dims(dims, tile_m)
    wdev = wdev if wdev is not None else weights_to_dev(case["w"])
    if case.get("shared_gate") is not None:
        wdev = dict(wdev, shared_gate=dev(case["shared_gate"]))
    logits = dev(case["logits"])
    x = dev(case["x"])
    r = B.alloc_routing(dm)
    ws = B.alloc_workspace(dm)
    y = torch.empty((dims.T, dims.d), dtype=torch.int16, device="cuda")
    if poison:  # NaN pattern: any element the kernels fail to write shows up
        y.fill_(0x7FC1)
        for t in r.values():
            t.fill_(-7)
    if mode == "layer":
        B.moe_layer(dm, logits, x, wdev, r, y, ws)
    else:
        B.moe_route(dm, logits, r, ws)
        B.moe_ffn(dm, x, wdev, r, y, ws)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in r.items()}
    out["y_bits"] = host_u16(y)
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


def check_y(case, g, ref_route, tokens=None):
    """y against the oracle on all tokens, or on the listed ones."""
    dims = case["dims"]
    y_ref = oracle.ffn(dims, case["x"], case["w"], ref_route["ids"], ref_route["w"], tokens=tokens,
                       shared_gate=case.get("shared_gate"))
    y = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    assert np.all(np.isfinite(g["y"])), "unwritten or non-finite outputs"
    err = float(np.abs(y - y_ref).max())
    tol = y_tolerance(y_ref)
    assert err <= tol, f"max|y - y_ref| = {err} > {tol}"
    return err, tol


def sample_tokens(case, ref_route, n_random=32, seed=0):
    """Tokens for a sampled comparison at full size: the first and last few,
    tokens of the most and least loaded non-empty experts, and random ones."""
    T = case["dims"].T
    ids = ref_route["ids"]
    counts = ref_route["counts"]
    pick = set(range(min(4, T))) | set(range(max(0, T - 4), T))
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    cold = int(nz[np.argmin(counts[nz])])
    for e in (hot, cold):
        toks = np.nonzero((ids == e).any(1))[0]
        pick |= set(int(t) for t in toks[:4]) | set(int(t) for t in toks[-4:])
    rng = np.random.default_rng(seed)
    pick |= set(int(t) for t in rng.choice(T, size=min(n_random, T), replace=False))
    return sorted(pick)
