"""Whole-matrix fp64 attention for tiny shapes -- TEST INFRASTRUCTURE ONLY.

An independent second route to the same definition as ``fa_oracle.c``: build
the full Q_S x KV_S score matrix per head, exclude masked and beyond-length
keys, take a row softmax, multiply by V (FlashAttn operator guide, function
description; developer guide 1.5-1.7 for masks, LSE and RowInvalid).  Pure
numpy; O(Q_S * KV_S) memory, so only for the small pin grids.
"""
from __future__ import annotations

import numpy as np


def _decode(bits, dtype):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def attention(prob, q, k, v):
    """Return out (q layout) and lse [B, QN, QS], both fp64."""
    B, QN, KVN, QS, KVS, D = prob.B, prob.QN, prob.KVN, prob.QS, prob.KVS, prob.D
    g = QN // KVN
    Q, K, V = _decode(q, prob.dtype), _decode(k, prob.dtype), _decode(v, prob.dtype)
    if prob.layout == "BSND":  # to [B, N, S, D]
        Q, K, V = (x.transpose(0, 2, 1, 3) for x in (Q, K, V))
    out = np.zeros((B, QN, QS, D))
    lse = np.full((B, QN, QS), np.inf)
    i_idx = np.arange(QS)[:, None]
    j_idx = np.arange(KVS)[None, :]
    for b in range(B):
        L = KVS if prob.lens is None else int(np.clip(prob.lens[b], 0, KVS))
        for n1 in range(QN):
            keep = np.broadcast_to(j_idx < L, (QS, KVS)).copy()
            if prob.mask_mode == "causal":
                keep &= ~(j_idx > i_idx)
            elif prob.mask_mode == "bool":
                st = prob.mask_strides
                flat = prob.mask.reshape(-1)
                idx = b * st[0] + n1 * st[1] + i_idx * st[2] + j_idx * st[3]
                keep &= flat[idx] == 0
            Kh = np.where(keep.any(axis=0)[:, None], K[b, n1 // g], 0.0)
            Vh = np.where(keep.any(axis=0)[:, None], V[b, n1 // g], 0.0)
            S = prob.scale * (Q[b, n1] @ Kh.T)
            S = np.where(keep, S, -np.inf)
            m = S.max(axis=1, initial=-np.inf)
            live = np.isfinite(m)
            E = np.where(keep, np.exp(S - np.where(live, m, 0.0)[:, None]), 0.0)
            l = E.sum(axis=1)
            o = E @ Vh
            out[b, n1, live] = o[live] / l[live, None]
            lse[b, n1, live] = np.log(l[live]) + m[live]
    if prob.layout == "BSND":
        out = out.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(out), lse
