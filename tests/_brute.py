"""Independent brute-force formulations used to pin the oracle (tests only).

Nothing here is shared with the oracle or the GPU library: dequantisation is
vectorised numpy on the raw bytes, routing is a full stable argsort, and the
MoE layer is a dense evaluation of every expert combined with a gate vector
that is zero outside the top-k.
"""
from __future__ import annotations

import numpy as np


def np_dequant(m: np.ndarray) -> np.ndarray:
    """uint8 [..., nb, 18] canonical blocks -> fp64 [..., nb*32]."""
    m = np.asarray(m, np.uint8)
    d = m[..., :2].copy().view("<f2")[..., 0].astype(np.float64)
    qs = m[..., 2:].astype(np.int64)
    q = np.concatenate([qs & 0xF, qs >> 4], axis=-1)  # [..., nb, 32]
    w = (q - 8).astype(np.float64) * d[..., None]
    return w.reshape(m.shape[:-2] + (m.shape[-2] * 32,))


def np_route(z: np.ndarray, k: int):
    """Top-k by a full stable sort of -z (ties: lower id), softmax over the chosen."""
    z = np.asarray(z, np.float32)
    order = np.argsort(-z.astype(np.float64), axis=-1, kind="stable")
    ids = order[..., :k].astype(np.int32)
    zs = np.take_along_axis(z.astype(np.float64), ids, axis=-1)
    ez = np.exp(zs - zs.max(axis=-1, keepdims=True))
    return ids, ez / ez.sum(axis=-1, keepdims=True)


def dense_moe(gates_q, ups_q, downs_q, x, z, k):
    """Evaluate every expert densely and combine with a dense gate vector.

    gates_q/ups_q [E][F][H/32][18], downs_q [E][H][F/32][18]; x fp64 [T][H];
    z fp32 [T][E]. Returns y fp64 [T][H].
    """
    Wg = np_dequant(gates_q)  # [E][F][H]
    Wu = np_dequant(ups_q)
    Wd = np_dequant(downs_q)  # [E][H][F]
    T = x.shape[0]
    E = Wg.shape[0]
    ids, w = np_route(z, k)
    gate_vec = np.zeros((T, E))
    for t in range(T):
        gate_vec[t, ids[t]] = w[t]
    g = np.einsum("efh,th->tef", Wg, x)
    u = np.einsum("efh,th->tef", Wu, x)
    h = g / (1.0 + np.exp(-g)) * u
    ye = np.einsum("ehf,tef->teh", Wd, h)  # every expert's output
    return np.einsum("te,teh->th", gate_vec, ye)
