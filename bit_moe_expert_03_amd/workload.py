"""Seeded synthetic inputs for the MoE FFN layer.

This module only draws numbers: it holds none of the layer's arithmetic (no
dequantisation, routing or FFN math), so both the HIP path and the CPU oracle
can take their inputs from it without sharing any of the method.

Shapes follow the model the pages describe (Qwen3.6-35B-A3B: 8 of 256 experts
plus one shared expert per token, groupwise affine 4-bit weights; page
"Perplexity's Lily Beats MLX-LM...", section "What Lily actually does", and
page "Perplexity Open Sources Lily: Rust & Metal Engine for Qwen3.6", bullet
list).  The pages give no tensor sizes; the five presets below are the
workloads this library is measured and checked on.

Recipe (every tensor has its own PCG64 stream seeded by
``SeedSequence([seed, index, tensor_id])``):

* activations x: N(0, 1) rounded to bf16 (round-to-nearest-even);
* router W_r: fp32 N(0, 1/d), shape [d, E];
* logits: the fp64 sum x . W_r (plus an optional per-expert bias) rounded once
  to fp32 -- the router projection is the caller's job, so it is an input here;
* Zipf bias: rank r_e = a seeded permutation of 1..E, bias_e = -ln r_e, so that
  softmax(bias) is exactly a Zipf(1) law over the experts;
* 4-bit codes: uniform on 0..15 (two codes per byte, uniform random bytes);
* scales: U[0.005, 0.02] rounded to bf16; biases: -8 * scale (exact in bf16).

Weight layout (shared with the C ABI): a matrix W of shape [N_out][K_in] is
stored as codes q[N_out][K_in/2] (element 2m in the low nibble of byte m,
element 2m+1 in the high nibble) plus bf16 scale and bias arrays
[N_out][K_in/G]; routed experts are stacked expert-major.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Dims:
    """Layer shape: T tokens, hidden d, E experts, top-k, expert width F,
    shared-expert width Fs, quantisation group G (along the input dim)."""

    T: int
    d: int
    E: int
    k: int
    F: int
    Fs: int
    G: int

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


# Named workloads (tiny, decode, prefill 512, skewed prefill 4096, long prefill).
CONFIGS: Dict[str, Dims] = {
    "c0_tiny": Dims(T=16, d=256, E=16, k=2, F=128, Fs=128, G=32),
    "c1_decode": Dims(T=1, d=2048, E=256, k=8, F=512, Fs=512, G=64),
    "c2_prefill512": Dims(T=512, d=2048, E=256, k=8, F=512, Fs=512, G=64),
    "c3_prefill4096_zipf": Dims(T=4096, d=2048, E=256, k=8, F=512, Fs=512, G=64),
    "c4_prefill32768": Dims(T=32768, d=2048, E=256, k=8, F=512, Fs=512, G=64),
}
ZIPF_CONFIGS = {"c3_prefill4096_zipf"}
SEED_OF = {name: i for i, name in enumerate(CONFIGS)}
DECODE_WEIGHT_SETS = 40  # distinct layer weight sets rotated by the decode workload

# tensor ids of the per-tensor seed streams
_TID = {
    "gate": 1, "up": 2, "down": 3, "sgate": 4, "sup": 5, "sdown": 6,
    "x": 10, "w_router": 11, "zipf": 12,
}
MATS = ("gate", "up", "down", "sgate", "sup", "sdown")


def _rng(seed: int, index: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index, tid])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def mat_shape(dims: Dims, name: str):
    """(experts, N_out, K_in) of one weight matrix; experts = 0 for shared."""
    E, d, F, Fs = dims.E, dims.d, dims.F, dims.Fs
    return {
        "gate": (E, F, d), "up": (E, F, d), "down": (E, d, F),
        "sgate": (0, Fs, d), "sup": (0, Fs, d), "sdown": (0, d, Fs),
    }[name]


def make_qmat(dims: Dims, name: str, seed: int, index: int = 0) -> Dict[str, np.ndarray]:
    """One packed matrix: {'q': uint8 [..,N,K/2], 's': uint16 [..,N,K/G], 'b': same}."""
    ne, n, kin = mat_shape(dims, name)
    lead = (ne,) if ne else ()
    rng = _rng(seed, index, _TID[name])
    nbytes = (ne or 1) * n * (kin // 2)
    q = np.frombuffer(rng.bytes(nbytes), dtype=np.uint8).reshape(lead + (n, kin // 2)).copy()
    s = rng.uniform(0.005, 0.02, size=lead + (n, kin // dims.G)).astype(np.float32)
    s_bits = to_bf16_bits(s)
    b_bits = to_bf16_bits(bf16_bits_to_f32(s_bits) * np.float32(-8.0))
    return {"q": q, "s": s_bits, "b": b_bits}


def make_weights(dims: Dims, seed: int, index: int = 0) -> Dict[str, Dict[str, np.ndarray]]:
    """All six packed matrices of one layer weight set."""
    return {m: make_qmat(dims, m, seed, index) for m in MATS}


def make_x(dims: Dims, seed: int, index: int = 0) -> np.ndarray:
    """Activations as bf16 bits, [T, d]."""
    x = _rng(seed, index, _TID["x"]).standard_normal((dims.T, dims.d), dtype=np.float32)
    return to_bf16_bits(x)


def make_router(dims: Dims, seed: int) -> np.ndarray:
    """Router projection W_r, fp32 [d, E], N(0, 1/d)."""
    w = _rng(seed, 0, _TID["w_router"]).standard_normal((dims.d, dims.E))
    return (w / np.sqrt(dims.d)).astype(np.float32)


def zipf_bias(E: int, seed: int) -> np.ndarray:
    """Per-expert bias -ln(rank) with a seeded rank permutation: softmax of it
    is Zipf(s=1) over the experts."""
    ranks = _rng(seed, 0, _TID["zipf"]).permutation(E) + 1
    return -np.log(ranks.astype(np.float64))


def make_logits(x_bits: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits fp32 [T, E]: fp64 x . W_r (+ bias), rounded once to fp32."""
    xf = bf16_bits_to_f32(x_bits).astype(np.float64)
    lg = xf @ w_router.astype(np.float64)
    if bias is not None:
        lg = lg + bias[None, :]
    return lg.astype(np.float32)


def make_case(name_or_dims, seed: Optional[int] = None, index: int = 0,
              zipf: Optional[bool] = None, weights: bool = True) -> dict:
    """Complete seeded input of one workload: dims, x, logits and weights."""
    if isinstance(name_or_dims, str):
        dims = CONFIGS[name_or_dims]
        seed = SEED_OF[name_or_dims] if seed is None else seed
        zipf = (name_or_dims in ZIPF_CONFIGS) if zipf is None else zipf
    else:
        dims = name_or_dims
        seed = 0 if seed is None else seed
        zipf = bool(zipf)
    x = make_x(dims, seed, index)
    wr = make_router(dims, seed)
    bias = zipf_bias(dims.E, seed) if zipf else None
    case = {"dims": dims, "seed": seed, "x": x, "logits": make_logits(x, wr, bias)}
    if weights:
        case["w"] = make_weights(dims, seed, index)
    return case



# ---- decode attention over grouped KV heads (the pages' second decode workload)

@dataclasses.dataclass(frozen=True)
class AttnDims:
    """One decode token: Hq query heads, Hkv KV heads (Hq = 8 Hkv: eight query
    heads share one KV head), head dimension D, L cached tokens."""

    Hq: int
    Hkv: int
    D: int
    L: int


# The pages name the sharing (8 query heads per KV head) and the contexts
# (4K in their benchmarks, 32K for the packing figure, up to 128K); the head
# counts and dimension below are this library's choice.
ATTN_CONFIGS: Dict[str, AttnDims] = {
    "attn_L4096": AttnDims(Hq=32, Hkv=4, D=128, L=4096),
    "attn_L32768": AttnDims(Hq=32, Hkv=4, D=128, L=32768),
    "attn_L131072": AttnDims(Hq=32, Hkv=4, D=128, L=131072),
}
_ATTN_TID = {"q": 20, "k": 21, "v": 22}


def make_attn_case(name_or_dims, seed: int = 7, index: int = 0) -> dict:
    """q [Hq][D] and the K, V caches [Hkv][L][D]: N(0, 1) rounded to bf16."""
    dims = ATTN_CONFIGS[name_or_dims] if isinstance(name_or_dims, str) else name_or_dims
    out = {"dims": dims, "seed": seed}
    shapes = {"q": (dims.Hq, dims.D), "k": (dims.Hkv, dims.L, dims.D), "v": (dims.Hkv, dims.L, dims.D)}
    for name, shape in shapes.items():
        out[name] = to_bf16_bits(_rng(seed, index, _ATTN_TID[name]).standard_normal(shape, dtype=np.float32))
    return out
