"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Routing outputs and dequantised weights: bit-exact.  Routing weights: within
1e-6 of the oracle's fp64 softmax and summing to 1 within 1e-6.  Layer output
y (bf16): max|y - y_ref| <= 1e-2 max|y_ref| + 1e-3 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_moe_expert_03_amd import binding as B
from bit_moe_expert_03_amd import workload as wl
from gpu_util import (bf16_to_f64, check_routing, check_y, dev, host_u16, run, tile_tokens,
                      weights_to_dev)

pytestmark = pytest.mark.gpu

# shapes the oracle finishes in seconds that span several tiles and ragged tails
SMALL = {
    "ragged_T37_E16_k4": (wl.Dims(T=37, d=128, E=16, k=4, F=64, Fs=128, G=32), False),
    "T300_E16_k4_G64": (wl.Dims(T=300, d=256, E=16, k=4, F=128, Fs=128, G=64), False),
    "T70_E8_k3_G128": (wl.Dims(T=70, d=256, E=8, k=3, F=128, Fs=128, G=128), False),
    "k_equals_E": (wl.Dims(T=9, d=64, E=4, k=4, F=64, Fs=64, G=32), False),
    "E1_k1": (wl.Dims(T=33, d=64, E=1, k=1, F=64, Fs=64, G=64), False),
    "T2_smallest_gemm": (wl.Dims(T=2, d=128, E=8, k=2, F=64, Fs=64, G=32), False),
    "zipf_T500_E64_k6": (wl.Dims(T=500, d=128, E=64, k=6, F=64, Fs=64, G=32), True),
    "T1_small_decode": (wl.Dims(T=1, d=256, E=16, k=4, F=128, Fs=192, G=64), False),
    # small batches (2 <= T <= 32, T k <= 512) take the matrix-vector kernels
    "T5_small_batch": (wl.Dims(T=5, d=256, E=16, k=4, F=128, Fs=192, G=64), False),
    "T16_small_batch": (wl.Dims(T=16, d=256, E=16, k=4, F=128, Fs=192, G=64), False),
    "T32_k16_batch_limit": (wl.Dims(T=32, d=128, E=64, k=16, F=64, Fs=64, G=32), False),
    "T33_over_T_limit": (wl.Dims(T=33, d=128, E=16, k=2, F=64, Fs=64, G=32), False),
    "T8_k64_batch_limit": (wl.Dims(T=8, d=128, E=64, k=64, F=64, Fs=64, G=32), False),
    "T8_k65_over_limit": (wl.Dims(T=8, d=128, E=80, k=65, F=64, Fs=64, G=32), False),
    # many rows per expert: several full 128-row tiles per expert,
    # widths that are not multiples of 128 and odd K-step counts
    "T1000_E4_k2_pairs": (wl.Dims(T=1000, d=128, E=4, k=2, F=192, Fs=64, G=64), False),
    "T600_E2_k1_G128_pairs": (wl.Dims(T=600, d=256, E=2, k=1, F=128, Fs=128, G=128), False),
    # expert counts that are not multiples of 4 (logit rows not 16-byte
    # aligned: the router GEMM stores them value by value), with the router's
    # K split into two ranges (d = 1024) and without (d = 256)
    "T37_E30_d1024_ksplit": (wl.Dims(T=37, d=1024, E=30, k=4, F=64, Fs=64, G=64), False),
    "T37_E13_k3": (wl.Dims(T=37, d=256, E=13, k=3, F=64, Fs=64, G=32), False),
    # many experts with one or two rows next to experts with more (the tail
    # of a skewed batch: one-row tiles on the matrix cores), at d = 2048,
    # F = 192, G = 128, and with down blocks chained over column blocks
    "fewrow_T40_E128_k2": (wl.Dims(T=40, d=256, E=128, k=2, F=128, Fs=64, G=32), False),
    "fewrow_T36_E64_k4_d2048": (wl.Dims(T=36, d=2048, E=64, k=4, F=64, Fs=64, G=64), False),
    "fewrow_T48_E96_k2_F192": (wl.Dims(T=48, d=1024, E=96, k=2, F=192, Fs=128, G=64), False),
    "fewrow_T40_E128_k2_G128": (wl.Dims(T=40, d=256, E=128, k=2, F=128, Fs=128, G=128), False),
}


@pytest.fixture(scope="module")
def cases():
    return {}


def _case(name):
    if name in wl.CONFIGS:
        return wl.make_case(name)
    dims, zipf = SMALL[name]
    return wl.make_case(dims, seed=100 + list(SMALL).index(name), zipf=zipf)


# ------------------------------------------------------------------ dequant

def test_dequant_bit_exact():
    rng = np.random.default_rng(1)
    for rows, cols, G in ((64, 256, 32), (512, 2048, 64), (96, 512, 128)):
        q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
        s = wl.to_bf16_bits(rng.uniform(-2, 2, (rows, cols // G)).astype(np.float32))
        b = wl.to_bf16_bits(rng.uniform(-30, 30, (rows, cols // G)).astype(np.float32))
        out = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
        B.moe_dequant(dev(q), dev(s), dev(b), rows, cols, G, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), oracle.dequant_bf16(q, s, b, rows, cols, G))


def test_dequant_workload_weights_bit_exact():
    c = wl.make_case("c2_prefill512")
    d = c["dims"]
    for m, (rows, cols) in (("gate", (d.F, d.d)), ("down", (d.d, d.F))):
        q, s, b = (c["w"][m][f][3] for f in ("q", "s", "b"))  # expert 3
        out = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
        B.moe_dequant(dev(q), dev(s), dev(b), rows, cols, d.G, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), oracle.dequant_bf16(q, s, b, rows, cols, d.G))


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_route_bit_exact_workloads(name):
    c = wl.make_case(name, weights=False)
    dm = B.make_dims(c["dims"])
    r = B.alloc_routing(dm)
    ws = B.alloc_workspace(dm)
    B.moe_route(dm, dev(c["logits"]), r, ws)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    g["tile_m"], g["max_tiles"] = B.moe_tile_m(dm), B.moe_max_tiles(dm)
    check_routing(c, g)


@pytest.mark.parametrize("tile_m", [32, 64, 128])
def test_route_tie_heavy_and_signed_zero(tile_m):
    rng = np.random.default_rng(tile_m)
    dims = wl.Dims(T=777, d=64, E=256, k=8, F=64, Fs=64, G=32)
    L = rng.integers(-2, 3, (dims.T, dims.E)).astype(np.float32)
    L[::3] *= 0.0  # rows of signed zeros: -0.0 and +0.0 must tie
    L[1::3] = np.where(rng.random((len(L[1::3]), dims.E)) < 0.5, -0.0, L[1::3])
    c = {"dims": dims, "logits": L}
    dm = B.make_dims(dims, tile_m)
    r = B.alloc_routing(dm)
    B.moe_route(dm, dev(L), r, B.alloc_workspace(dm))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    g["tile_m"], g["max_tiles"] = tile_m, B.moe_max_tiles(dm)
    check_routing(c, g)


def test_route_empty_batch():
    dims = wl.Dims(T=0, d=64, E=8, k=2, F=64, Fs=64, G=32)
    dm = B.make_dims(dims)
    r = B.alloc_routing(dm)
    for t in r.values():
        t.fill_(-7)
    B.moe_route(dm, torch.empty((0, 8), device="cuda"), r, B.alloc_workspace(dm))
    torch.cuda.synchronize()
    assert np.all(r["counts"].cpu().numpy() == 0)
    assert np.all(r["offsets"].cpu().numpy() == 0)
    assert int(r["num_tiles"].cpu()[0]) == 0


# ------------------------------------------------------------------ layer

@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_shapes_all_tokens(name):
    c = _case(name)
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)


# the largest dimensions the entry points take: d, F and Fs up to 16384 and
# k = E = 256, on the decode path (T <= 32) and on the GEMM path (T = 33)
MAXDIMS = {
    "max_d_decode": wl.Dims(T=1, d=16384, E=256, k=8, F=64, Fs=64, G=64),
    "max_d_gemm": wl.Dims(T=33, d=16384, E=256, k=8, F=64, Fs=64, G=64),
    "max_F_decode": wl.Dims(T=1, d=128, E=4, k=2, F=16384, Fs=16384, G=128),
    "max_F_gemm": wl.Dims(T=33, d=256, E=4, k=2, F=16384, Fs=16384, G=128),
    "k_eq_E_256_decode": wl.Dims(T=2, d=64, E=256, k=256, F=64, Fs=64, G=64),
    "k_eq_E_256_gemm": wl.Dims(T=33, d=64, E=256, k=256, F=64, Fs=64, G=64),
}


@pytest.mark.parametrize("name", list(MAXDIMS))
def test_layer_maximum_dims_all_tokens(name):
    dims = MAXDIMS[name]
    c = wl.make_case(dims, seed=400 + list(MAXDIMS).index(name))
    g = run(c)
    ref = check_routing(c, g)
    check_y(c, g, ref)


@pytest.mark.parametrize("name", [n for n in SMALL if SMALL[n][0].T >= 2])
def test_layer_small_shapes_tile128(name):
    """Every small shape with 128-row tiles (the four-sub-tile GEMM bodies)."""
    c = _case(name)
    g = run(c, tile_m=128)
    ref = check_routing(c, g)
    check_y(c, g, ref)


def test_layer_tiny_config_all_tokens():
    c = wl.make_case("c0_tiny")
    for tile_m in (0, 32, 64, 128):
        g = run(c, tile_m=tile_m)
        ref = check_routing(c, g)
        check_y(c, g, ref, label=f"c0_tiny tile_m={tile_m}")


@pytest.mark.parametrize("tile_m", [0, 32, 128])
def test_layer_prefill512_all_tokens(tile_m):
    c = wl.make_case("c2_prefill512")
    g = run(c, tile_m=tile_m, mode="split" if tile_m == 32 else "layer")
    ref = check_routing(c, g)
    check_y(c, g, ref, key="c2_prefill512", label=f"c2_prefill512 tile_m={tile_m}")


def test_layer_prefill4096_zipf_all_tokens():
    c = wl.make_case("c3_prefill4096_zipf")
    g = run(c)
    ref = check_routing(c, g)
    check_y(c, g, ref, key="c3_prefill4096_zipf", label="c3_prefill4096_zipf")


def test_tile_heights_give_identical_bits_full_size():
    """T = 4096 Zipf: y at every tile height is bit-identical (the tile
    height changes which rows share a workgroup, never the order of a sum)."""
    c = wl.make_case("c3_prefill4096_zipf")
    ys = {tm: run(c, tile_m=tm)["y_bits"] for tm in (32, 64, 128)}
    for tm in (32, 64):
        np.testing.assert_array_equal(ys[tm], ys[128], err_msg=f"tile_m={tm}")


def test_layer_prefill32768_every_tile():
    """T = 32768: y on the tokens that put a row into every routed and every
    shared tile the GEMM kernels run (first and last row of each tile)."""
    c = wl.make_case("c4_prefill32768")
    g = run(c)
    ref = check_routing(c, g)
    toks = tile_tokens(c, ref, g["tile_m"])
    check_y(c, g, ref, tokens=toks, key="c4_prefill32768", label="c4_prefill32768 every tile")


# Down GEMM with chained column blocks (one block runs several 256-column
# blocks of its tile as one pipeline): chosen through moe_dims.down_nc on
# shapes with d a multiple of 256 and F = Fs = 64 * 2^n.
CHAINED = {
    "chain_T300_d1024_F128": wl.Dims(T=300, d=1024, E=16, k=4, F=128, Fs=128, G=64),
    "chain_T90_d1024_F256_G32": wl.Dims(T=90, d=1024, E=8, k=2, F=256, Fs=256, G=32),
    "chain_T40_d512_F512_G128": wl.Dims(T=40, d=512, E=4, k=3, F=512, Fs=512, G=128),
    "chain_fewrow_T40_d1024_E128": wl.Dims(T=40, d=1024, E=128, k=2, F=128, Fs=128, G=64),
}


@pytest.mark.parametrize("nc", [2, 4])
@pytest.mark.parametrize("name", list(CHAINED))
def test_down_chained_column_blocks(name, nc):
    dims = CHAINED[name]
    if (dims.d // 256) % nc:
        pytest.skip("chain length must divide the column-block count")
    c = wl.make_case(dims, seed=200 + list(CHAINED).index(name))
    for tile_m in (0, 32, 128):
        g = run(c, tile_m=tile_m, down_nc=nc)
        ref = check_routing(c, g)
        check_y(c, g, ref)


def test_down_chain_length_does_not_change_bits():
    """The chain length changes the schedule only: each output element sees
    the same MFMA sequence, so y is bit-identical for every length."""
    dims = CHAINED["chain_T300_d1024_F128"]
    c = wl.make_case(dims, seed=210)
    ys = {nc: run(c, down_nc=nc)["y_bits"] for nc in (1, 2, 4)}
    np.testing.assert_array_equal(ys[1], ys[2])
    np.testing.assert_array_equal(ys[1], ys[4])


@pytest.mark.parametrize("nc", [1, 2, 8])
def test_down_chain_lengths_full_size(nc):
    """T = 4096 Zipf at every chain length (the default picks one): y on
    every token that has a row in some tile, and bit-identical to the
    default schedule."""
    c = wl.make_case("c3_prefill4096_zipf")
    g = run(c, down_nc=nc)
    ref = check_routing(c, g)
    check_y(c, g, ref, tokens=tile_tokens(c, ref, g["tile_m"]), key="c3_prefill4096_zipf",
            label=f"c3_prefill4096_zipf down_nc={nc}")
    np.testing.assert_array_equal(g["y_bits"], run(c)["y_bits"])


GATED = ["ragged_T37_E16_k4", "T300_E16_k4_G64", "T70_E8_k3_G128", "T1_small_decode", "T5_small_batch",
         "zipf_T500_E64_k6"]


@pytest.mark.parametrize("name", GATED)
def test_layer_gated_shared_expert(name):
    """Shared expert scaled by sigmoid(x . g) per token: both paths (GEMM
    combine, decode down kernel), fused and split calls, two tile heights."""
    c = dict(_case(name))
    d = c["dims"].d
    rng = np.random.default_rng(7)
    c["shared_gate"] = wl.to_bf16_bits((rng.standard_normal(d) / np.sqrt(d)).astype(np.float32))
    for mode, tile_m in (("layer", 0), ("split", 128)):
        g = run(c, mode=mode, tile_m=tile_m)
        ref = check_routing(c, g)
        check_y(c, g, ref)


def test_decode_gated_shared_expert_full_size():
    c = dict(wl.make_case("c1_decode", index=3))
    rng = np.random.default_rng(8)
    c["shared_gate"] = wl.to_bf16_bits((rng.standard_normal(c["dims"].d) / np.sqrt(c["dims"].d)).astype(np.float32))
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)


def test_prefill_gated_shared_expert_all_tokens():
    c = dict(wl.make_case("c2_prefill512"))
    rng = np.random.default_rng(9)
    c["shared_gate"] = wl.to_bf16_bits((rng.standard_normal(c["dims"].d) / np.sqrt(c["dims"].d)).astype(np.float32))
    g = run(c)
    ref = check_routing(c, g)
    check_y(c, g, ref, label="c2_prefill512 gated shared expert")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_tie_heavy_logits(seed):
    """T = 1 with logits in {-1, -0, 0, 1}: most of the top 8 are exact ties.
    Every routed wave of the decode kernel ranks the experts itself, so each
    must break ties to the lower id as the oracle does (a wrong expert shows
    in y as well as in the routing outputs of the fused path)."""
    dims = wl.Dims(T=1, d=256, E=64, k=8, F=128, Fs=128, G=64)
    c = wl.make_case(dims, seed=300 + seed)
    rng = np.random.default_rng(seed)
    L = rng.integers(-1, 2, (1, dims.E)).astype(np.float32)
    L[0, rng.random(dims.E) < 0.3] = -0.0
    c["logits"] = L
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)


@pytest.mark.parametrize("T", [2, 3, 5, 8, 9, 16, 31, 32])
def test_small_batch_full_size(T):
    """Few-token batches at the workload's layer shape: every token of every
    slot, routing outputs bit-exact in both the fused and the split call."""
    dims = wl.Dims(T=T, d=2048, E=256, k=8, F=512, Fs=512, G=64)
    c = wl.make_case(dims, seed=400 + T, index=T)
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)


@pytest.mark.parametrize("T,seed", [(6, 0), (6, 1), (32, 2)])
def test_small_batch_tie_heavy_logits(T, seed):
    """Logits in {-1, -0, 0, 1}: tokens share experts and tie inside the top
    8, so the batch's stable sorted order and tiles are exercised (T = 32:
    up to 32 rows of one expert in one tile)."""
    dims = wl.Dims(T=T, d=256, E=32, k=8, F=128, Fs=128, G=64)
    c = wl.make_case(dims, seed=500 + seed)
    rng = np.random.default_rng(50 + seed)
    L = rng.integers(-1, 2, (dims.T, dims.E)).astype(np.float32)
    L[rng.random((dims.T, dims.E)) < 0.3] = -0.0
    c["logits"] = L
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)


@pytest.mark.parametrize("index", [0, 1, 39])
def test_decode_full_size(index):
    c = wl.make_case("c1_decode", index=index)
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref, label=f"c1_decode set {index} {mode}")


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("name", ["c0_tiny", "c1_decode", "T300_E16_k4_G64"])
def test_deterministic(name):
    c = _case(name)
    wdev = weights_to_dev(c["w"])
    a = run(c, wdev=wdev)
    b = run(c, wdev=wdev)
    for k in ("topk_ids", "topk_w", "perm", "y_bits"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("name", ["c0_tiny", "c1_decode", "T300_E16_k4_G64"])
def test_doubling_down_scales_doubles_y(name):
    c = _case(name)
    g = run(c)
    c2 = dict(c)
    c2["w"] = {m: dict(v) for m, v in c["w"].items()}
    for m in ("down", "sdown"):
        for f in ("s", "b"):
            c2["w"][m][f] = wl.to_bf16_bits(2.0 * bf16_to_f64(c["w"][m][f]).astype(np.float32))
    g2 = run(c2)
    np.testing.assert_array_equal(g2["y"], 2.0 * g["y"])


def test_token_permutation_permutes_rows():
    c = _case("T300_E16_k4_G64")
    g = run(c)
    p = np.random.default_rng(0).permutation(c["dims"].T)
    c2 = dict(c)
    c2["x"] = np.ascontiguousarray(c["x"][p])
    c2["logits"] = np.ascontiguousarray(c["logits"][p])
    g2 = run(c2)
    np.testing.assert_array_equal(g2["y_bits"], g["y_bits"][p])


def test_expert_relabelling_leaves_y_unchanged():
    c = _case("T300_E16_k4_G64")
    g = run(c)
    p = np.random.default_rng(1).permutation(c["dims"].E)
    c2 = dict(c)
    c2["w"] = {m: ({f: np.ascontiguousarray(a[p]) for f, a in v.items()} if m in ("gate", "up", "down") else v)
               for m, v in c["w"].items()}
    c2["logits"] = np.ascontiguousarray(c["logits"][:, p])
    g2 = run(c2)
    np.testing.assert_array_equal(g2["y_bits"], g["y_bits"])


# ------------------------------------------------------------------ launch forms

@pytest.mark.parametrize("name", ["c0_tiny", "T1_small_decode", "T5_small_batch"])
def test_timed_entry_point_matches_and_times(name):
    c = _case(name)
    dims = c["dims"]
    dm = B.make_dims(dims)
    g = run(c)
    wdev = weights_to_dev(c["w"])
    nk = B.moe_layer_kernels(dm)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    r = B.alloc_routing(dm)
    y = torch.empty((dims.T, dims.d), dtype=torch.int16, device="cuda")
    B.moe_layer_timed(dm, dev(c["logits"]), dev(c["x"]), wdev, r, y, B.alloc_workspace(dm),
                      [e.cuda_event for e in evs])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(y), g["y_bits"])
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(nk)]
    assert all(t > 0 for t in times), times
    with pytest.raises(B.MoeError):  # too few events: rejected before any launch
        B.moe_layer_timed(dm, dev(c["logits"]), dev(c["x"]), wdev, r, y, B.alloc_workspace(dm),
                          [e.cuda_event for e in evs[:-1]])


@pytest.mark.parametrize("name", ["c0_tiny", "T1_small_decode", "T5_small_batch", "T300_E16_k4_G64"])
def test_graph_replays_match_eager(name):
    c = _case(name)
    dims = c["dims"]
    dm = B.make_dims(dims)
    eager = run(c)
    wdev = weights_to_dev(c["w"])
    lg, x = dev(c["logits"]), dev(c["x"])
    r = B.alloc_routing(dm)
    ws = B.alloc_workspace(dm)
    y = torch.empty((dims.T, dims.d), dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=s):
            B.moe_layer(dm, lg, x, wdev, r, y, ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(0x7FC1)
        r["perm"].fill_(-7)
        gr.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(y), eager["y_bits"], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(r["perm"].cpu().numpy(), eager["perm"])
        # the program's own eager work between replays
        B.moe_layer(dm, lg, x, wdev, B.alloc_routing(dm), torch.empty_like(y), B.alloc_workspace(dm))
        torch.cuda.synchronize()


# ------------------------------------------------------------------ router projection

def _route_x(c, with_bias):
    """moe_router_pack + moe_route_x on the case's activations and router."""
    dims = c["dims"]
    dm = B.make_dims(dims)
    wr = wl.make_router(dims, c["seed"])
    bias = wl.zipf_bias(dims.E, c["seed"]).astype(np.float32) if with_bias else None
    packed = torch.empty(B.moe_router_packed_bytes(dm) // 2, dtype=torch.int16, device="cuda")
    B.moe_router_pack(dm, dev(wr), packed)
    logits = torch.full((dims.T, dims.E), float("nan"), dtype=torch.float32, device="cuda")
    r = B.alloc_routing(dm)
    for t in r.values():
        t.fill_(-7)
    B.moe_route_x(dm, dev(c["x"]), packed, dev(bias) if bias is not None else None, logits, r,
                  B.alloc_workspace(dm))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    g["tile_m"], g["max_tiles"] = B.moe_tile_m(dm), B.moe_max_tiles(dm)
    return logits.cpu().numpy(), g, wr, bias


ROUTER_CASES = [("c0_tiny", False), ("c1_decode", False), ("c2_prefill512", False),
                ("c3_prefill4096_zipf", True), ("ragged_T37_E16_k4", False), ("T5_small_batch", True),
                ("T8_k65_over_limit", False), ("T37_E30_d1024_ksplit", True), ("T37_E13_k3", True)]


@pytest.mark.parametrize("name,with_bias", ROUTER_CASES, ids=[n for n, _ in ROUTER_CASES])
def test_route_x_logits_and_routing(name, with_bias):
    """Router logits from the packed bf16 hi/lo router on the matrix cores:
    within the bound of the split (|W - hi - lo| <= 2^-17 |W|) and of fp32
    accumulation, 2^-14 sum_i |x_i W_ie| + 1e-6, against the fp64 oracle;
    the routing of those logits bit-exact against the oracle's routing of
    the same logits (near-ties may order differently from the fp64 logits,
    so the routing is compared on the GPU's own)."""
    c = dict(_case(name) if name in SMALL else wl.make_case(name, weights=False))
    L, g, wr, bias = _route_x(c, with_bias)
    L_ref = oracle.router_logits(c["x"], wr, bias)
    bound = 2.0 ** -14 * (np.abs(bf16_to_f64(c["x"])) @ np.abs(wr.astype(np.float64))) + 1e-6
    assert np.all(np.isfinite(L)), "unwritten logits"
    assert np.all(np.abs(L - L_ref) <= bound), float(np.max(np.abs(L - L_ref) / bound))
    check_routing(dict(c, logits=L), g)


def test_route_x_then_ffn_matches_oracle():
    """The layer from the activations: moe_route_x, then moe_ffn on its
    routing, against the oracle's layer on the GPU's logits."""
    c = dict(_case("T300_E16_k4_G64"))
    L, g_route, wr, _ = _route_x(c, False)
    c2 = dict(c, logits=L)
    g = run(c2, mode="split")  # moe_route on the same logits, then moe_ffn
    for k in ("topk_ids", "perm", "inv_perm", "counts", "offsets"):
        np.testing.assert_array_equal(g[k], g_route[k])
    ref = check_routing(c2, g)
    check_y(c2, g, ref)


def test_route_x_empty_batch():
    """T = 0: nothing to project or route; the call succeeds and writes the
    empty histogram and tile count."""
    dims = wl.Dims(T=0, d=256, E=16, k=2, F=128, Fs=128, G=32)
    dm = B.make_dims(dims)
    packed = torch.zeros(B.moe_router_packed_bytes(dm) // 2, dtype=torch.int16, device="cuda")
    r = B.alloc_routing(dm)
    for t in r.values():
        t.fill_(-7)
    B.moe_route_x(dm, torch.empty((0, dims.d), dtype=torch.int16, device="cuda"), packed, None,
                  torch.empty((0, dims.E), dtype=torch.float32, device="cuda"), r, B.alloc_workspace(dm))
    torch.cuda.synchronize()
    assert np.all(r["counts"].cpu().numpy() == 0)
    assert np.all(r["offsets"].cpu().numpy() == 0)
    assert int(r["num_tiles"].cpu()[0]) == 0


def test_small_batch_gated_shared_expert_full_size():
    """A 4-token batch at the workload's layer shape with the shared expert
    gated by sigmoid(x_t . g) per token (block 0 forms the four gates)."""
    dims = wl.Dims(T=4, d=2048, E=256, k=8, F=512, Fs=512, G=64)
    c = dict(wl.make_case(dims, seed=404, index=4))
    rng = np.random.default_rng(10)
    c["shared_gate"] = wl.to_bf16_bits((rng.standard_normal(dims.d) / np.sqrt(dims.d)).astype(np.float32))
    for mode in ("layer", "split"):
        g = run(c, mode=mode)
        ref = check_routing(c, g)
        check_y(c, g, ref)
