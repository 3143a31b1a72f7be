"""CPU oracle of the MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do: the two implementations share no code, only the seeded inputs of
``bit_moe_expert_03_amd.workload``.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, one token at a time);
this module compiles it with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_I32P = ctypes.POINTER(ctypes.c_int32)
_F64P = ctypes.POINTER(ctypes.c_double)
_F32P = ctypes.POINTER(ctypes.c_float)
_U16P = ctypes.POINTER(ctypes.c_uint16)
_U8P = ctypes.POINTER(ctypes.c_uint8)


class _OMat(ctypes.Structure):
    _fields_ = [("q", _U8P), ("s", _U16P), ("b", _U16P)]


class _OWeights(ctypes.Structure):
    _fields_ = [(n, _OMat) for n in ("gate", "up", "down", "sgate", "sup", "sdown")]


def build(force: bool = True, extra_flags: Sequence[str] = (), out: Optional[str] = None) -> str:
    """Compile moe_oracle.c into a shared library (gcc, OpenMP, no fp contraction).

    ``extra_flags`` lets a test compile a variant (e.g. with a planted mistake)
    into ``out`` without touching the default library."""
    out = out or _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               *extra_flags, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _declare(lib):
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_dequant_exact.argtypes = [_U8P, _U16P, _U16P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _F64P]
    lib.oracle_dequant_bf16.argtypes = [_U8P, _U16P, _U16P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _U16P]
    lib.oracle_topk.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _F32P, _I32P, _F64P]
    lib.oracle_counting_sort.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _I32P, _I32P, _I32P, _I32P, _I32P]
    lib.oracle_block_map.argtypes = [ctypes.c_int, _I32P, _I32P, ctypes.c_int, ctypes.c_int, _I32P, _I32P, _I32P]
    lib.oracle_block_map.restype = ctypes.c_int
    lib.oracle_ffn.argtypes = [ctypes.c_int] * 7 + [_U16P, ctypes.POINTER(_OWeights), _U16P, _I32P, _F64P,
                                                    _I32P, ctypes.c_int, _F64P]
    lib.oracle_router_logits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _U16P, _F32P, _F32P, _F64P]
    lib.oracle_gqa_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _U16P, _U16P, _U16P,
                                      _F64P]
    return lib


def load(path: Optional[str] = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray, ptype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ptype)


def threads(lib=None) -> int:
    return (lib or load()).oracle_threads()


def dequant_exact(q, s, b, rows: int, cols: int, G: int, lib=None) -> np.ndarray:
    """Exact s*q + b of a [rows][cols] packed matrix, fp64."""
    lib = lib or load()
    q, s, b = (np.ascontiguousarray(a) for a in (q, s, b))
    out = np.empty((rows, cols), np.float64)
    lib.oracle_dequant_exact(_p(q, _U8P), _p(s, _U16P), _p(b, _U16P), rows, cols, G, _p(out, _F64P))
    return out


def dequant_bf16(q, s, b, rows: int, cols: int, G: int, lib=None) -> np.ndarray:
    """bf16 bits of bf16_rne(fp32_rne(s*q + b)), [rows][cols] uint16."""
    lib = lib or load()
    q, s, b = (np.ascontiguousarray(a) for a in (q, s, b))
    out = np.empty((rows, cols), np.uint16)
    lib.oracle_dequant_bf16(_p(q, _U8P), _p(s, _U16P), _p(b, _U16P), rows, cols, G, _p(out, _U16P))
    return out


def topk(logits: np.ndarray, k: int, lib=None):
    """(ids int32 [T,k], weights fp64 [T,k]) of the k best experts per token."""
    lib = lib or load()
    L = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib.oracle_topk(T, E, k, _p(L, _F32P), _p(ids, _I32P), _p(w, _F64P))
    return ids, w


def counting_sort(ids: np.ndarray, E: int, lib=None):
    """(counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]) of the assignments."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    lib.oracle_counting_sort(T, E, k, _p(ids, _I32P), _p(counts, _I32P), _p(offsets, _I32P),
                             _p(perm, _I32P), _p(inv, _I32P))
    return counts, offsets, perm, inv


def block_map(counts: np.ndarray, offsets: np.ndarray, tile_m: int, max_tiles: int, lib=None):
    """(tile_expert, tile_row0, tile_rows) arrays of length num_tiles."""
    lib = lib or load()
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    te = np.full(max_tiles, -1, np.int32)
    tr = np.full(max_tiles, -1, np.int32)
    tn = np.full(max_tiles, -1, np.int32)
    n = lib.oracle_block_map(len(counts), _p(counts, _I32P), _p(offsets, _I32P), tile_m, max_tiles,
                             _p(te, _I32P), _p(tr, _I32P), _p(tn, _I32P))
    if n < 0:
        raise ValueError("block map needs more than max_tiles tiles")
    return te[:n].copy(), tr[:n].copy(), tn[:n].copy()


def route(logits: np.ndarray, k: int, tile_m: int, max_tiles: Optional[int] = None, lib=None) -> dict:
    """Every routing output for one batch of logits."""
    T, E = logits.shape
    ids, w = topk(logits, k, lib)
    counts, offsets, perm, inv = counting_sort(ids, E, lib)
    if max_tiles is None:
        max_tiles = -(-T * k // tile_m) + min(E, T * k)
    te, tr, tn = block_map(counts, offsets, tile_m, max_tiles, lib)
    return {"ids": ids, "w": w, "counts": counts, "offsets": offsets, "perm": perm, "inv_perm": inv,
            "tile_expert": te, "tile_row0": tr, "tile_rows": tn, "num_tiles": len(te)}


def router_logits(x_bits: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None,
                  lib=None) -> np.ndarray:
    """fp64 router logits x W_r (+ bias): x bf16 bits [T][d], W_r fp32 [d][E]."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    W = np.ascontiguousarray(w_router, dtype=np.float32)
    T, d = x.shape
    E = W.shape[1]
    assert W.shape[0] == d
    L = np.empty((T, E), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib.oracle_router_logits(T, d, E, _p(x, _U16P), _p(W, _F32P), None if b is None else _p(b, _F32P), _p(L, _F64P))
    return L


def gqa_decode(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, lib=None) -> np.ndarray:
    """fp64 decode attention of one token: q bf16 bits [Hq][D], k and v bf16
    bits [Hkv][L][D]; query head h reads KV head h // (Hq // Hkv)."""
    lib = lib or load()
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    Hq, D = q.shape
    Hkv, L, D2 = k.shape
    assert D2 == D and v.shape == k.shape and Hq % Hkv == 0
    out = np.empty((Hq, D), np.float64)
    lib.oracle_gqa_decode(Hq, Hkv, D, L, _p(q, _U16P), _p(k, _U16P), _p(v, _U16P), _p(out, _F64P))
    return out


def ffn(dims, x_bits: np.ndarray, weights: dict, ids: np.ndarray, w: np.ndarray,
        tokens: Optional[Sequence[int]] = None, shared_gate=None,
        lib=None) -> np.ndarray:
    """y (fp64) for all tokens, or for the listed token indices: [len, d].
    shared_gate: optional bf16 bits [d]; the shared expert's output is then
    scaled by sigmoid(x_t . shared_gate) per token (else by 1)."""
    lib = lib or load()
    keep = []

    def mat(name):
        m = weights[name]
        arrs = [np.ascontiguousarray(m[f]) for f in ("q", "s", "b")]
        keep.extend(arrs)
        return _OMat(_p(arrs[0], _U8P), _p(arrs[1], _U16P), _p(arrs[2], _U16P))

    W = _OWeights(*[mat(n) for n in ("gate", "up", "down", "sgate", "sup", "sdown")])
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    if tokens is None:
        tok_p, ntok = None, dims.T
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        keep.append(tok)
        tok_p, ntok = _p(tok, _I32P), len(tok)
    y = np.empty((ntok, dims.d), np.float64)
    sg_p = None
    if shared_gate is not None:
        sg = np.ascontiguousarray(shared_gate, dtype=np.uint16)
        assert sg.shape == (dims.d,)
        keep.append(sg)
        sg_p = _p(sg, _U16P)
    lib.oracle_ffn(dims.T, dims.d, dims.E, dims.k, dims.F, dims.Fs, dims.G, _p(x_bits, _U16P),
                   ctypes.byref(W), sg_p, _p(ids, _I32P), _p(w, _F64P), tok_p, ntok, _p(y, _F64P))
    return y
