"""Pins of the CPU oracle: each check raises AssertionError on a mismatch.

Every check takes the oracle library handle, so the same checks run on the
real oracle (tests/test_oracle_pins.py) and on copies with a planted mistake
(tests/test_oracle_mutations.py), which must fail at least one of them.

What pins what (none of them re-types the oracle's own formula):
* hand-worked fixtures under tests/golden/ (nibble order, group index, affine
  decode, bf16 ties, routing ties and signed zeros, scatter, tiles);
* library routines: numpy's stable argsort (top-k order, scatter), bincount and
  cumsum (histogram, scan), scipy's softmax and expit, torch's bf16 cast and
  float64 SwiGLU via torch.nn.functional.silu;
* a dense brute force over all experts (tests/bruteforce.py);
* closed forms (b = -8 s gives s (q - 8); integer weights give integer sums)
  and invariants (doubling down-projection scales doubles y; relabelling the
  experts leaves y unchanged).
"""
import json
import os

import numpy as np
import scipy.special
import torch

import oracle
from bit_moe_expert_03_amd import workload as wl
from bruteforce import bf16_to_f64, brute_layer, swiglu_mlp, topk_argsort, unpack_dense

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def torch_bf16_bits(v):
    """fp64 -> fp32 (numpy, RNE) -> bf16 (torch, RNE) bits."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ dequant

def check_packing_fixture(lib):
    f = _golden("packing_example.json")
    q = np.array(f["q_bytes"], np.uint8)
    s = np.array(f["s_bf16"], np.uint16)
    b = np.array(f["b_bf16"], np.uint16)
    w = oracle.dequant_exact(q, s, b, f["rows"], f["cols"], f["G"], lib=lib)
    np.testing.assert_array_equal(w, np.array(f["expected_w"]))
    wb = oracle.dequant_bf16(q, s, b, f["rows"], f["cols"], f["G"], lib=lib)
    np.testing.assert_array_equal(wb, torch_bf16_bits(np.array(f["expected_w"])))
    # the codes in the fixture are the nibbles of the bytes, low nibble first
    codes = np.array(f["codes"])
    np.testing.assert_array_equal(codes[:, 0::2], q & 15)
    np.testing.assert_array_equal(codes[:, 1::2], q >> 4)


def check_rounding_fixture(lib):
    f = _golden("packing_example.json")
    for c in f["rounding_cases"]:
        # one group of two elements; the case's code sits in element 0
        q = np.array([[c["code"]]], np.uint8)
        s = np.array([[c["s_bf16"]]], np.uint16)
        b = np.array([[c["b_bf16"]]], np.uint16)
        w = oracle.dequant_exact(q, s, b, 1, 2, 2, lib=lib)
        assert w[0, 0] == c["exact"], (c, w)
        wb = oracle.dequant_bf16(q, s, b, 1, 2, 2, lib=lib)
        assert int(wb[0, 0]) == c["bf16"], (c, hex(int(wb[0, 0])))


def check_dequant_closed_form(lib):
    """b = -8 s gives exactly s (q - 8) for every code and every bf16 scale
    with exponent in [-30, 30]; the bf16 form equals torch's RNE cast."""
    exps = np.arange(127 - 30, 127 + 31, dtype=np.uint16)
    mant = np.arange(128, dtype=np.uint16)
    s_bits = ((exps[:, None] << 7) | mant[None, :]).ravel()
    n = s_bits.size
    s_val = bf16_to_f64(s_bits)
    b_bits = torch_bf16_bits(-8.0 * s_val)
    G = 16
    codes = np.tile(np.arange(16, dtype=np.uint8), (n, 1))  # one group of 16 codes per row
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w = oracle.dequant_exact(q, s_bits[:, None], b_bits[:, None], n, G, G, lib=lib)
    want = s_val[:, None] * (np.arange(16)[None, :] - 8.0)
    np.testing.assert_array_equal(w, want)
    wb = oracle.dequant_bf16(q, s_bits[:, None], b_bits[:, None], n, G, G, lib=lib)
    np.testing.assert_array_equal(wb, torch_bf16_bits(want))


def check_dequant_general_rounding(lib):
    """Arbitrary bf16 scale/bias pairs: the bf16 form is torch's RNE cast of
    the fp32 rounding of the exact value (brute-force unpack)."""
    rng = np.random.default_rng(7)
    rows, cols, G = 512, 64, 32
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    s = wl.to_bf16_bits(rng.uniform(-3, 3, (rows, cols // G)).astype(np.float32) *
                        np.float32(2.0) ** rng.integers(-6, 6, (rows, cols // G)).astype(np.float32))
    b = wl.to_bf16_bits(rng.uniform(-50, 50, (rows, cols // G)).astype(np.float32))
    dense = unpack_dense(q, s, b, G)
    np.testing.assert_array_equal(oracle.dequant_exact(q, s, b, rows, cols, G, lib=lib), dense)
    np.testing.assert_array_equal(oracle.dequant_bf16(q, s, b, rows, cols, G, lib=lib), torch_bf16_bits(dense))


# ------------------------------------------------------------------ routing

def check_route_fixture(lib):
    f = _golden("route_example.json")
    L = np.array(f["logits"], np.float32)
    assert np.signbit(L[1, 0]) and not np.signbit(L[1, 1])
    r = oracle.route(L, f["k"], f["tile_m"], lib=lib)
    np.testing.assert_array_equal(r["ids"], f["ids"])
    np.testing.assert_allclose(r["w"], f["weights"], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r["counts"], f["counts"])
    np.testing.assert_array_equal(r["offsets"], f["offsets"])
    np.testing.assert_array_equal(r["perm"], f["perm"])
    np.testing.assert_array_equal(r["inv_perm"], f["inv_perm"])
    tiles = np.stack([r["tile_expert"], r["tile_row0"], r["tile_rows"]], 1)
    np.testing.assert_array_equal(tiles, f["tiles"])
    r1 = oracle.route(L, f["k"], 1, lib=lib)
    tiles1 = np.stack([r1["tile_expert"], r1["tile_row0"], r1["tile_rows"]], 1)
    np.testing.assert_array_equal(tiles1, f["tiles_tile_m_1"])


def _logit_cases():
    rng = np.random.default_rng(11)
    yield rng.standard_normal((64, 256)).astype(np.float32), 8
    yield rng.integers(-3, 4, (64, 256)).astype(np.float32), 8  # heavy ties
    z = rng.integers(-1, 2, (32, 16)).astype(np.float32) * 0.0  # only +0 / -0
    yield np.where(rng.random((32, 16)) < 0.5, -z, z).astype(np.float32), 5
    yield rng.standard_normal((16, 16)).astype(np.float32), 16  # k = E
    yield rng.standard_normal((16, 7)).astype(np.float32), 1


def check_topk_vs_argsort(lib):
    for L, k in _logit_cases():
        ids, w = oracle.topk(L, k, lib=lib)
        np.testing.assert_array_equal(ids, topk_argsort(L, k))
        sel = np.take_along_axis(L.astype(np.float64), ids, axis=1)
        np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
        # every selected logit >= every unselected one
        mask = np.zeros(L.shape, bool)
        np.put_along_axis(mask, ids, True, axis=1)
        lo_sel = np.where(mask, L, np.inf).min(1)
        hi_uns = np.where(mask, -np.inf, L).max(1)
        assert np.all(lo_sel >= hi_uns)


def check_weights_special(lib):
    rng = np.random.default_rng(5)
    L = rng.standard_normal((8, 12)).astype(np.float32)
    ids, w = oracle.topk(L, 12, lib=lib)  # k = E: the full softmax, reordered
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, axis=1), rtol=1e-14)
    _, w1 = oracle.topk(L, 1, lib=lib)  # k = 1: weight exactly 1
    assert np.all(w1 == 1.0)


def check_counting_sort(lib):
    rng = np.random.default_rng(3)
    for T, E, k in ((1, 256, 8), (33, 16, 2), (512, 256, 8), (100, 5, 5)):
        L = rng.standard_normal((T, E)).astype(np.float32)
        L[:, : E // 3] += 2.0  # skew: some experts popular, some empty
        ids, _ = oracle.topk(L, k, lib=lib)
        counts, offsets, perm, inv = oracle.counting_sort(ids, E, lib=lib)
        np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert counts.sum() == T * k and offsets[-1] == T * k
        np.testing.assert_array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
        np.testing.assert_array_equal(inv[perm], np.arange(T * k))
        np.testing.assert_array_equal(np.sort(perm), np.arange(T * k))


def check_block_map(lib):
    rng = np.random.default_rng(9)
    for trial in range(20):
        E = int(rng.integers(1, 40))
        counts = rng.integers(0, 300, E).astype(np.int32)
        counts[rng.random(E) < 0.3] = 0
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        tile_m = int(rng.choice([1, 16, 32, 64, 128]))
        max_tiles = -(-int(counts.sum()) // tile_m) + E
        te, tr, tn = oracle.block_map(counts, offsets, tile_m, max_tiles, lib=lib)
        assert len(te) == int(np.sum(-(-counts // tile_m)))
        covered = np.zeros(int(counts.sum()), np.int32)
        for e, r0, n in zip(te, tr, tn):
            assert 1 <= n <= tile_m
            assert offsets[e] <= r0 and r0 + n <= offsets[e + 1]
            covered[r0:r0 + n] += 1
        assert np.all(covered == 1)
        assert np.all(np.diff(te) >= 0) and np.all(np.diff(tr) > 0)


# ------------------------------------------------------------------ FFN

SMALL_SHAPES = [
    wl.Dims(T=5, d=64, E=4, k=2, F=32, Fs=32, G=32),
    wl.Dims(T=3, d=64, E=8, k=8, F=32, Fs=64, G=16),
    wl.Dims(T=7, d=128, E=6, k=3, F=64, Fs=128, G=64),
]


def check_ffn_bruteforce(lib):
    cases = [wl.make_case("c0_tiny")] + [wl.make_case(dm, seed=20 + i) for i, dm in enumerate(SMALL_SHAPES)]
    for c in cases:
        dims = c["dims"]
        r = oracle.route(c["logits"], dims.k, 16, lib=lib)
        y = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], lib=lib)
        yb, ids_b, _ = brute_layer(dims, c["x"], c["w"], c["logits"])
        np.testing.assert_array_equal(r["ids"], ids_b)
        err = np.abs(y - yb).max() / np.abs(yb).max()
        assert err <= 1e-12, (dims, err)
        # a subset of tokens gives the same rows
        sub = [dims.T - 1, 0]
        ys = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=sub, lib=lib)
        np.testing.assert_array_equal(ys, y[sub])


def check_ffn_single_expert_torch(lib):
    """E = k = 1: the layer is two dense SwiGLU MLPs (torch, fp64, F.silu)."""
    dims = wl.Dims(T=6, d=64, E=1, k=1, F=32, Fs=64, G=32)
    c = wl.make_case(dims, seed=31)
    r = oracle.route(c["logits"], 1, 8, lib=lib)
    assert np.all(r["w"] == 1.0)
    y = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], lib=lib)
    W = {m: torch.from_numpy(unpack_dense(c["w"][m]["q"], c["w"][m]["s"], c["w"][m]["b"], dims.G))
         for m in wl.MATS}
    X = torch.from_numpy(bf16_to_f64(c["x"]))

    def mlp(g, u, dn):
        return (torch.nn.functional.silu(X @ g.T) * (X @ u.T)) @ dn.T

    want = mlp(W["gate"][0], W["up"][0], W["down"][0]) + mlp(W["sgate"], W["sup"], W["sdown"])
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-12)


def check_ffn_integer(lib):
    """s = 1, b = 0 and integer x: gate/up sums are exact integers (numpy
    int64 matmul).  The down matrix is the identity (code 1 on the diagonal)
    and the shared expert is zero (s = b = 0), so y = silu(g) * u."""
    dims = wl.Dims(T=4, d=32, E=1, k=1, F=32, Fs=32, G=16)
    rng = np.random.default_rng(2)
    xi = rng.integers(-4, 5, (dims.T, dims.d))
    x_bits = wl.to_bf16_bits(xi.astype(np.float32))
    one, zero = np.uint16(0x3F80), np.uint16(0)

    def qmat(codes, s_bits, b_bits):
        q = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
        shp = codes.shape[:-1] + (codes.shape[-1] // dims.G,)
        return {"q": q, "s": np.full(shp, s_bits, np.uint16), "b": np.full(shp, b_bits, np.uint16)}

    cg = rng.integers(0, 16, (1, dims.F, dims.d)).astype(np.uint8)
    cu = rng.integers(0, 16, (1, dims.F, dims.d)).astype(np.uint8)
    eye = np.eye(dims.d, dtype=np.uint8)[None]
    W = {"gate": qmat(cg, one, zero), "up": qmat(cu, one, zero), "down": qmat(eye, one, zero),
         "sgate": qmat(cg[0], zero, zero), "sup": qmat(cu[0], zero, zero), "sdown": qmat(eye[0], zero, zero)}
    ids = np.zeros((dims.T, 1), np.int32)
    w = np.ones((dims.T, 1))
    y = oracle.ffn(dims, x_bits, W, ids, w, lib=lib)
    g = xi.astype(np.int64) @ cg[0].astype(np.int64).T
    u = xi.astype(np.int64) @ cu[0].astype(np.int64).T
    want = g * scipy.special.expit(g.astype(np.float64)) * u
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-12)


def check_ffn_metamorphic(lib):
    c = wl.make_case("c0_tiny")
    dims = c["dims"]
    r = oracle.route(c["logits"], dims.k, 16, lib=lib)
    y = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], lib=lib)
    # doubling every scale and bias of both down projections doubles y exactly
    W2 = {m: dict(v) for m, v in c["w"].items()}
    for m in ("down", "sdown"):
        for f in ("s", "b"):
            W2[m][f] = torch_bf16_bits(2.0 * bf16_to_f64(c["w"][m][f]))
    y2 = oracle.ffn(dims, c["x"], W2, r["ids"], r["w"], lib=lib)
    np.testing.assert_array_equal(y2, 2.0 * y)
    # relabelling the experts (weights and logit columns together) changes nothing
    p = np.random.default_rng(4).permutation(dims.E)
    W3 = {m: ({f: a[p] for f, a in v.items()} if m in ("gate", "up", "down") else v) for m, v in c["w"].items()}
    L3 = np.ascontiguousarray(c["logits"][:, p])
    r3 = oracle.route(L3, dims.k, 16, lib=lib)
    np.testing.assert_array_equal(p[r3["ids"]], r["ids"])
    y3 = oracle.ffn(dims, c["x"], W3, r3["ids"], r3["w"], lib=lib)
    np.testing.assert_array_equal(y3, y)


def check_ffn_shared_gate(lib):
    """Shared-expert gate: brute force (numpy dot, scipy expit) on small
    shapes, and the limits of one token with g = +-64 x_0: the gate reads 1
    (y equals the ungated layer exactly) and 0 (routed experts only); with
    g = 0 it reads 1/2, halfway between the two."""
    for i, dims in enumerate(SMALL_SHAPES):
        c = wl.make_case(dims, seed=40 + i)
        rng = np.random.default_rng(50 + i)
        g = wl.to_bf16_bits((rng.standard_normal(dims.d) / np.sqrt(dims.d)).astype(np.float32))
        r = oracle.route(c["logits"], dims.k, 16, lib=lib)
        y = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], shared_gate=g, lib=lib)
        yb, _, _ = brute_layer(dims, c["x"], c["w"], c["logits"], shared_gate=g)
        err = np.abs(y - yb).max() / np.abs(yb).max()
        assert err <= 1e-12, (dims, err)
    dims = SMALL_SHAPES[0]
    c = wl.make_case(dims, seed=45)
    r = oracle.route(c["logits"], dims.k, 16, lib=lib)
    x0 = bf16_to_f64(c["x"][0])
    y_free = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=[0], lib=lib)
    y_one = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=[0], lib=lib,
                       shared_gate=torch_bf16_bits(64.0 * x0))
    y_zero = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=[0], lib=lib,
                        shared_gate=torch_bf16_bits(-64.0 * x0))
    y_half = oracle.ffn(dims, c["x"], c["w"], r["ids"], r["w"], tokens=[0], lib=lib,
                        shared_gate=np.zeros(dims.d, np.uint16))
    np.testing.assert_array_equal(y_one, y_free)
    assert np.abs(y_one - y_zero).max() > 1e-3 * np.abs(y_one).max()  # the shared part is not negligible
    np.testing.assert_allclose(y_half, 0.5 * (y_one + y_zero), rtol=1e-12, atol=1e-12)


def check_router_logits_vs_matmul(lib):
    """Router logits against numpy's fp64 matrix product of the decoded
    activations (d != E, so a transposed operand shows) plus the bias."""
    rng = np.random.default_rng(31)
    T, d, E = 5, 96, 40
    x = wl.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    ref = bf16_to_f64(x) @ W.astype(np.float64) + bias.astype(np.float64)
    got = oracle.router_logits(x, W, bias, lib=lib)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    got0 = oracle.router_logits(x, W, None, lib=lib)
    np.testing.assert_allclose(got0, ref - bias.astype(np.float64), rtol=1e-12, atol=1e-12)


def check_router_logits_identity(lib):
    """Closed form: with W_r the first E columns of the identity (d >= E),
    token t's logits are its first E activations, exactly."""
    rng = np.random.default_rng(32)
    T, d, E = 3, 64, 48
    x = wl.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = np.eye(d, E, dtype=np.float32)
    got = oracle.router_logits(x, W, None, lib=lib)
    assert np.array_equal(got, bf16_to_f64(x)[:, :E])


# ---- decode attention over grouped KV heads

def _attn_case(Hq, Hkv, D, L, seed):
    return wl.make_attn_case(wl.AttnDims(Hq=Hq, Hkv=Hkv, D=D, L=L), seed=seed)


def check_attn_torch_sdpa(lib):
    """Against torch's scaled_dot_product_attention in float64 on the CPU, the
    KV heads repeated over their groups of query heads (repeat_interleave:
    query head h reads KV head h // G)."""
    for Hq, Hkv, D, L in ((16, 2, 16, 37), (8, 1, 64, 300), (32, 4, 8, 5)):
        c = _attn_case(Hq, Hkv, D, L, 41)
        G = Hq // Hkv
        q = torch.from_numpy(bf16_to_f64(c["q"])).view(1, Hq, 1, D)
        k = torch.from_numpy(bf16_to_f64(c["k"])).repeat_interleave(G, dim=0).view(1, Hq, L, D)
        v = torch.from_numpy(bf16_to_f64(c["v"])).repeat_interleave(G, dim=0).view(1, Hq, L, D)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).view(Hq, D).numpy()
        got = oracle.gqa_decode(c["q"], c["k"], c["v"], lib=lib)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def check_attn_closed_forms(lib):
    """q = 0: every score is 0, so o is the plain mean of the V rows; L = 1:
    o is that single V row exactly; one key with a score far above the rest
    takes all the weight (exp(-60) below fp64 resolution of the sum)."""
    c = _attn_case(16, 2, 32, 9, 42)
    zero = np.zeros_like(c["q"])
    got = oracle.gqa_decode(zero, c["k"], c["v"], lib=lib)
    means = bf16_to_f64(c["v"]).mean(axis=1)  # [Hkv][D]
    np.testing.assert_allclose(got, np.repeat(means, 8, axis=0), rtol=1e-13, atol=1e-14)
    c1 = _attn_case(16, 2, 32, 1, 43)
    got1 = oracle.gqa_decode(c1["q"], c1["k"], c1["v"], lib=lib)
    assert np.array_equal(got1, np.repeat(bf16_to_f64(c1["v"])[:, 0, :], 8, axis=0))
    # one dominant key: k_t* = 16 q_h for every t in the group, others 0 -> s_t* = 16 |q|^2 / sqrt(D)
    Hq, Hkv, D, L = 8, 1, 16, 6
    q = wl.to_bf16_bits(np.full((Hq, D), 1.0, np.float32))
    k = np.zeros((Hkv, L, D), np.uint16)
    k[0, 4] = wl.to_bf16_bits(np.full(D, 16.0, np.float32))
    v = _attn_case(Hq, Hkv, D, L, 44)["v"]
    got2 = oracle.gqa_decode(q, k, v, lib=lib)
    np.testing.assert_allclose(got2, np.repeat(bf16_to_f64(v)[:, 4, :], Hq, axis=0), rtol=0, atol=1e-12)


def check_attn_grouping_and_order(lib):
    """Each query head reads only its own KV head (constant V rows per KV head
    give constant outputs per group), and reversing the cached tokens leaves
    every output unchanged."""
    Hq, Hkv, D, L = 24, 3, 16, 11
    c = _attn_case(Hq, Hkv, D, L, 45)
    v = np.empty((Hkv, L, D), np.uint16)
    for g in range(Hkv):
        v[g] = wl.to_bf16_bits(np.full((L, D), float(g + 1), np.float32))
    got = oracle.gqa_decode(c["q"], c["k"], v, lib=lib)
    np.testing.assert_allclose(got, np.repeat(np.arange(1.0, Hkv + 1.0), Hq // Hkv)[:, None] * np.ones((1, D)),
                               rtol=1e-13)
    a = oracle.gqa_decode(c["q"], c["k"], c["v"], lib=lib)
    b = oracle.gqa_decode(c["q"], c["k"][:, ::-1].copy(), c["v"][:, ::-1].copy(), lib=lib)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


ALL_CHECKS = [
    check_packing_fixture, check_rounding_fixture, check_dequant_closed_form,
    check_dequant_general_rounding, check_route_fixture, check_topk_vs_argsort,
    check_weights_special, check_counting_sort, check_block_map, check_ffn_bruteforce,
    check_ffn_single_expert_torch, check_ffn_integer, check_ffn_metamorphic, check_ffn_shared_gate,
    check_router_logits_vs_matmul, check_router_logits_identity,
    check_attn_torch_sdpa, check_attn_closed_forms, check_attn_grouping_and_order,
]
