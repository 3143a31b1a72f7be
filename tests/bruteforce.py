"""Dense brute-force evaluation of the MoE layer (numpy, fp64), for tiny inputs.

It is deliberately a different computation from the oracle's: every token is
run through ALL experts as dense matrices (unpacked with vectorised numpy, not
per element), routing is numpy's stable argsort, the softmax and the sigmoid
come from scipy, and the mixture is a masked sum over every expert -- no
permutation, no per-expert grouping.  It pins the oracle on small shapes.
"""
import numpy as np
import scipy.special


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_dense(q, s, b, G):
    """[..., N, K/2] codes + [..., N, K/G] s/b -> dense fp64 [..., N, K]."""
    q = np.asarray(q)
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.float64)
    codes[..., 0::2] = q & 0x0F
    codes[..., 1::2] = q >> 4
    sf = np.repeat(bf16_to_f64(s), G, axis=-1)
    bf = np.repeat(bf16_to_f64(b), G, axis=-1)
    return codes * sf + bf


def topk_argsort(logits, k):
    """Top-k ids by numpy's stable sort of -logits (ties keep ascending id;
    -0.0 and +0.0 compare equal)."""
    L = np.asarray(logits, dtype=np.float64)
    return np.argsort(-L, axis=1, kind="stable")[:, :k]


def swiglu_mlp(X, Wg, Wu, Wd):
    """Dense SwiGLU MLP on rows of X: (silu(X Wg^T) * (X Wu^T)) Wd^T."""
    g = X @ Wg.T
    u = X @ Wu.T
    h = g * scipy.special.expit(g) * u
    return h @ Wd.T


def brute_layer(dims, x_bits, W, logits, shared_gate=None):
    """y [T, d] fp64 = gamma * shared(x) + sum over ALL experts of
    mask[t,e] * FFN_e(x); gamma = 1, or expit(x . g) per token with a gate
    vector g (bf16 bits [d])."""
    T, E, k, G = dims.T, dims.E, dims.k, dims.G
    X = bf16_to_f64(x_bits)
    ids = topk_argsort(logits, k)
    sel = np.take_along_axis(np.asarray(logits, np.float64), ids, axis=1)
    wts = scipy.special.softmax(sel, axis=1)
    mask = np.zeros((T, E))
    np.put_along_axis(mask, ids, wts, axis=1)
    Wg = unpack_dense(W["gate"]["q"], W["gate"]["s"], W["gate"]["b"], G)
    Wu = unpack_dense(W["up"]["q"], W["up"]["s"], W["up"]["b"], G)
    Wd = unpack_dense(W["down"]["q"], W["down"]["s"], W["down"]["b"], G)
    y = swiglu_mlp(X, unpack_dense(W["sgate"]["q"], W["sgate"]["s"], W["sgate"]["b"], G),
                   unpack_dense(W["sup"]["q"], W["sup"]["s"], W["sup"]["b"], G),
                   unpack_dense(W["sdown"]["q"], W["sdown"]["s"], W["sdown"]["b"], G))
    if shared_gate is not None:
        y = y * scipy.special.expit(X @ bf16_to_f64(shared_gate))[:, None]
    for e in range(E):
        y = y + mask[:, e:e + 1] * swiglu_mlp(X, Wg[e], Wu[e], Wd[e])
    return y, ids, wts
