"""ctypes binding of libmoe.so (include/moe.h), with the same function names.

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  PyTorch supplies device memory (``data_ptr()``) and the HIP
stream (``torch.cuda.current_stream().cuda_stream``), nothing else.  There is
no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_SHAPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
EXPORTS = ("moe_abi_version", "moe_tile_m", "moe_max_tiles", "moe_workspace_bytes", "moe_route",
           "moe_ffn", "moe_layer", "moe_layer_kernels", "moe_layer_timed", "moe_dequant",
           "moe_router_packed_bytes", "moe_router_pack", "moe_route_x", "moe_layer_noalloc",
           "moe_status_string", "moe_last_error", "moe_gqa_workspace_bytes", "moe_gqa_decode",
           "moe_gqa_decode_timed")
MATS = ("gate", "up", "down", "sgate", "sup", "sdown")


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"moe status {status}: {detail}")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "d", "E", "k", "F", "Fs", "G", "tile_m", "down_nc")]


class moe_attn_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("Hq", "Hkv", "D", "L")]


class moe_qmat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, moe_qmat) for n in MATS] + [("shared_gate", ctypes.c_void_p)]


ROUTING_FIELDS = ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm",
                  "tile_expert", "tile_row0", "tile_rows", "num_tiles")


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTING_FIELDS]


_lib = None


def lib():
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m bit_moe_expert_03_amd.build` "
                               "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.moe_abi_version.restype = ctypes.c_int32
        for f in ("moe_tile_m", "moe_layer_kernels"):
            getattr(L, f).restype = ctypes.c_int32
            getattr(L, f).argtypes = [P(moe_dims)]
        for f in ("moe_max_tiles", "moe_workspace_bytes", "moe_router_packed_bytes"):
            getattr(L, f).restype = ctypes.c_size_t
            getattr(L, f).argtypes = [P(moe_dims)]
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.moe_route.argtypes = [P(moe_dims), vp, P(moe_routing), vp, sz, vp]
        L.moe_ffn.argtypes = [P(moe_dims), vp, P(moe_weights), P(moe_routing), vp, vp, sz, vp]
        L.moe_layer.argtypes = [P(moe_dims), vp, vp, P(moe_weights), P(moe_routing), vp, vp, sz, vp]
        L.moe_layer_noalloc.argtypes = [P(moe_dims), vp, vp, P(moe_weights), P(moe_routing), vp, vp]
        L.moe_layer_timed.argtypes = [P(moe_dims), vp, vp, P(moe_weights), P(moe_routing), vp, vp, sz,
                                      vp, P(ctypes.c_void_p), ctypes.c_int32]
        L.moe_dequant.argtypes = [P(moe_qmat), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
        L.moe_router_pack.argtypes = [P(moe_dims), vp, vp, vp]
        L.moe_route_x.argtypes = [P(moe_dims), vp, vp, vp, vp, P(moe_routing), vp, sz, vp]
        L.moe_gqa_workspace_bytes.restype = ctypes.c_size_t
        L.moe_gqa_workspace_bytes.argtypes = [P(moe_attn_dims)]
        L.moe_gqa_decode.argtypes = [P(moe_attn_dims), vp, vp, vp, vp, vp, sz, vp]
        L.moe_gqa_decode_timed.argtypes = [P(moe_attn_dims), vp, vp, vp, vp, vp, sz, vp,
                                           P(ctypes.c_void_p), ctypes.c_int32]
        for f in ("moe_route", "moe_ffn", "moe_layer", "moe_layer_timed", "moe_dequant", "moe_router_pack",
                  "moe_route_x", "moe_layer_noalloc", "moe_gqa_decode", "moe_gqa_decode_timed"):
            getattr(L, f).restype = ctypes.c_int
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_dims(dims, tile_m: int = 0, down_nc: int = 0) -> moe_dims:
    """moe_dims from any object with T, d, E, k, F, Fs, G attributes; tile_m
    and down_nc are schedule fields (0: the library picks)."""
    return moe_dims(dims.T, dims.d, dims.E, dims.k, dims.F, dims.Fs, dims.G,
                    getattr(dims, "tile_m", 0) or tile_m, down_nc)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_tile_m(dims: moe_dims) -> int:
    return lib().moe_tile_m(ctypes.byref(dims))


def moe_max_tiles(dims: moe_dims) -> int:
    return lib().moe_max_tiles(ctypes.byref(dims))


def moe_workspace_bytes(dims: moe_dims) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(dims))


def weights_struct(w: Dict[str, Dict[str, torch.Tensor]]) -> moe_weights:
    """moe_weights from {'gate': {'q','s','b'}, ...} device tensors, plus an
    optional 'shared_gate' entry (bf16 bits [d]) for the gated shared expert."""
    sg = w.get("shared_gate")
    return moe_weights(*[moe_qmat(_ptr(w[m]["q"]), _ptr(w[m]["s"]), _ptr(w[m]["b"])) for m in MATS],
                       _ptr(sg) if sg is not None else None)


def routing_struct(r: Dict[str, torch.Tensor]) -> moe_routing:
    return moe_routing(*[_ptr(r[f]) for f in ROUTING_FIELDS])


def alloc_routing(dims: moe_dims, device="cuda") -> Dict[str, torch.Tensor]:
    """Device tensors for every routing output of these dims."""
    A = dims.T * dims.k
    mt = moe_max_tiles(dims)
    i32 = dict(dtype=torch.int32, device=device)
    return {
        "topk_ids": torch.empty((dims.T, dims.k), **i32),
        "topk_w": torch.empty((dims.T, dims.k), dtype=torch.float32, device=device),
        "counts": torch.empty(dims.E, **i32),
        "offsets": torch.empty(dims.E + 1, **i32),
        "perm": torch.empty(A, **i32),
        "inv_perm": torch.empty(A, **i32),
        "tile_expert": torch.empty(mt, **i32),
        "tile_row0": torch.empty(mt, **i32),
        "tile_rows": torch.empty(mt, **i32),
        "num_tiles": torch.empty(1, **i32),
    }


def alloc_workspace(dims: moe_dims, device="cuda") -> torch.Tensor:
    """Workspace of moe_workspace_bytes(dims), zero-filled before first use."""
    return torch.zeros(max(moe_workspace_bytes(dims), 256), dtype=torch.uint8, device=device)


def moe_route(dims: moe_dims, logits: torch.Tensor, routing: Dict[str, torch.Tensor],
              ws: torch.Tensor, stream=None):
    r = routing_struct(routing)
    _check(lib().moe_route(ctypes.byref(dims), _ptr(logits), ctypes.byref(r), _ptr(ws),
                           ws.numel(), _stream(stream)))


def moe_router_packed_bytes(dims: moe_dims) -> int:
    return lib().moe_router_packed_bytes(ctypes.byref(dims))


def moe_router_pack(dims: moe_dims, w_router: torch.Tensor, packed: torch.Tensor, stream=None):
    """w_router fp32 [d][E] -> packed bf16 hi/lo router (moe_router_packed_bytes bytes)."""
    _check(lib().moe_router_pack(ctypes.byref(dims), _ptr(w_router), _ptr(packed), _stream(stream)))


def moe_route_x(dims: moe_dims, x: torch.Tensor, packed: torch.Tensor, bias: Optional[torch.Tensor],
                logits: torch.Tensor, routing: Dict[str, torch.Tensor], ws: torch.Tensor, stream=None):
    """Router logits x W_r (+ bias) into `logits`, then the routing into `routing`."""
    r = routing_struct(routing)
    _check(lib().moe_route_x(ctypes.byref(dims), _ptr(x), _ptr(packed), _ptr(bias), _ptr(logits),
                             ctypes.byref(r), _ptr(ws), ws.numel(), _stream(stream)))


def moe_ffn(dims: moe_dims, x: torch.Tensor, weights, routing: Dict[str, torch.Tensor],
            y: torch.Tensor, ws: torch.Tensor, stream=None):
    w = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    r = routing_struct(routing)
    _check(lib().moe_ffn(ctypes.byref(dims), _ptr(x), ctypes.byref(w), ctypes.byref(r), _ptr(y),
                         _ptr(ws), ws.numel(), _stream(stream)))


def moe_layer(dims: moe_dims, logits: torch.Tensor, x: torch.Tensor, weights,
              routing: Dict[str, torch.Tensor], y: torch.Tensor, ws: torch.Tensor, stream=None):
    w = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    r = routing_struct(routing)
    _check(lib().moe_layer(ctypes.byref(dims), _ptr(logits), _ptr(x), ctypes.byref(w),
                           ctypes.byref(r), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def moe_layer_noalloc(dims: moe_dims, logits: torch.Tensor, x: torch.Tensor, weights,
                      routing: Dict[str, torch.Tensor], y: torch.Tensor, stream=None):
    """moe_layer on the library's own device scratch array (no workspace)."""
    w = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    r = routing_struct(routing)
    _check(lib().moe_layer_noalloc(ctypes.byref(dims), _ptr(logits), _ptr(x), ctypes.byref(w),
                                   ctypes.byref(r), _ptr(y), _stream(stream)))


def moe_layer_kernels(dims: moe_dims) -> int:
    return lib().moe_layer_kernels(ctypes.byref(dims))


def moe_layer_timed(dims: moe_dims, logits: torch.Tensor, x: torch.Tensor, weights,
                    routing: Dict[str, torch.Tensor], y: torch.Tensor, ws: torch.Tensor,
                    events, stream=None):
    """moe_layer plus events recorded around each kernel; `events` is a
    sequence of raw hipEvent_t handles (ints), at least moe_layer_kernels()+1."""
    w = weights if isinstance(weights, moe_weights) else weights_struct(weights)
    r = routing_struct(routing)
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().moe_layer_timed(ctypes.byref(dims), _ptr(logits), _ptr(x), ctypes.byref(w),
                                 ctypes.byref(r), _ptr(y), _ptr(ws), ws.numel(), _stream(stream),
                                 arr, len(events)))


def moe_dequant(q: torch.Tensor, s: torch.Tensor, b: torch.Tensor, rows: int, cols: int, G: int,
                out: torch.Tensor, stream=None):
    m = moe_qmat(_ptr(q), _ptr(s), _ptr(b))
    _check(lib().moe_dequant(ctypes.byref(m), rows, cols, G, _ptr(out), _stream(stream)))


def make_attn_dims(a) -> moe_attn_dims:
    """moe_attn_dims from any object with Hq, Hkv, D, L attributes."""
    return moe_attn_dims(a.Hq, a.Hkv, a.D, a.L)


def moe_gqa_workspace_bytes(dims: moe_attn_dims) -> int:
    return lib().moe_gqa_workspace_bytes(ctypes.byref(dims))


def alloc_gqa_workspace(dims: moe_attn_dims, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_gqa_workspace_bytes(dims), 256), dtype=torch.uint8, device=device)


def moe_gqa_decode(dims: moe_attn_dims, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   o: torch.Tensor, ws: torch.Tensor, stream=None):
    """o[h] = softmax(q[h] . k[h // 8] / sqrt(D)) v[h // 8]; bf16 bits in and out."""
    _check(lib().moe_gqa_decode(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws),
                                ws.numel(), _stream(stream)))


def moe_gqa_decode_timed(dims: moe_attn_dims, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         o: torch.Tensor, ws: torch.Tensor, events, stream=None):
    """moe_gqa_decode with events around its two kernels (at least 4 raw hipEvent_t handles)."""
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().moe_gqa_decode_timed(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws),
                                      ws.numel(), _stream(stream), arr, len(events)))
