"""The allocation-free entry point, moe_layer_noalloc, through the C ABI
against moe_layer with a caller-owned workspace: the same kernels in the
same order, so every output must be identical bit for bit.  Consecutive
calls of decreasing size share the library's one scratch array, so a later,
smaller call must not depend on what an earlier call left there."""
import numpy as np
import pytest
import torch

from bit_moe_expert_03_amd import binding as B
from bit_moe_expert_03_amd import workload as wl
from gpu_util import bf16_to_f64, check_routing, check_y, dev, host_u16, run, weights_to_dev

pytestmark = pytest.mark.gpu

ROUTING = ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm", "num_tiles")


def _noalloc(case):
    dims = case["dims"]
    dm = B.make_dims(dims)
    r = B.alloc_routing(dm)
    for t in r.values():
        t.fill_(-7)
    y = torch.full((dims.T, dims.d), 0x7FC1, dtype=torch.int16, device="cuda")  # NaN pattern
    B.moe_layer_noalloc(dm, dev(case["logits"]), dev(case["x"]), weights_to_dev(case["w"]), r, y)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in r.items()}
    out["y_bits"] = host_u16(y)
    return out


def _same(a, b, what):
    for k in ROUTING + ("y_bits",):
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")
    n = int(a["num_tiles"][0])
    for k in ("tile_expert", "tile_row0", "tile_rows"):
        np.testing.assert_array_equal(a[k][:n], b[k][:n], err_msg=f"{what}: {k}")


def test_noalloc_matches_layer_on_consecutive_calls():
    """T = 512 (about 31 of the 32 MiB of scratch), then smaller calls on the
    same scratch: T = 37, T = 16, T = 1 decode, and T = 512 again."""
    cases = [("T512", wl.make_case("c2_prefill512")),
             ("T37", wl.make_case(wl.Dims(T=37, d=128, E=16, k=4, F=64, Fs=128, G=32), seed=101)),
             ("T16", wl.make_case("c0_tiny")),
             ("T1", wl.make_case("c1_decode", index=5)),
             ("T512 again", wl.make_case("c2_prefill512"))]
    for name, c in cases:
        got = _noalloc(c)
        ref = run(c)  # moe_layer with its own workspace
        _same(got, ref, name)
    # and the small ones against the oracle directly
    for name, c in cases[1:4]:
        g = run(c)
        na = _noalloc(c)
        g.update(na)
        g["y"] = bf16_to_f64(na["y_bits"])
        check_y(c, g, check_routing(c, g), label=f"noalloc {name}")


def test_noalloc_rejects_dims_beyond_its_scratch():
    """T = 4096 needs about 213 MiB of workspace: refused before any launch."""
    c = wl.make_case("c3_prefill4096_zipf", weights=False)
    dims = c["dims"]
    dm = B.make_dims(dims)
    assert B.moe_workspace_bytes(dm) > B.NOALLOC_SCRATCH_BYTES
    r = B.alloc_routing(dm)
    y = torch.empty((dims.T, dims.d), dtype=torch.int16, device="cuda")
    w = {m: {f: torch.zeros(1, dtype=torch.int16, device="cuda") for f in ("q", "s", "b")} for m in wl.MATS}
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_noalloc(dm, dev(c["logits"]), dev(c["x"]), w, r, y)
    assert e.value.status == B.MOE_ERR_WORKSPACE
