"""Independent brute-force checks for the oracle (tests only).

Beam histories are simulated FORWARD by copying, the way a system that
treats each beam as an independent sequence does (the xGR technical summary,
section 1, describes that approach: every beam re-reads the prompt and
branching copies blocks).  Each beam's full key/value sequence is then
materialised and plain float64 softmax attention is applied with numpy.
Nothing here follows parent chains backwards, and nothing is shared with
the oracle's C code.
"""
from __future__ import annotations

import numpy as np

from generative_recommendation_beam_xattn_amd.workloads import bf16_bits_to_f32


def as_f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def histories(parent_idx: np.ndarray, step: int):
    """hist[r][b] = list of (level, slot) pairs, built level by level by copying."""
    R, S, BW = parent_idx.shape
    out = []
    for r in range(R):
        hist = [[(0, b)] for b in range(BW)]
        for t in range(1, step + 1):
            hist = [list(hist[int(parent_idx[r, t, b])]) + [(t, b)] for b in range(BW)]
        out.append(hist)
    return out


def attend(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
           scale=None):
    """out[r][b][h] = softmax(scale * K q) V over the materialised sequence."""
    q, sk, sv = as_f64(q), as_f64(shared_k), as_f64(shared_v)
    uk, uv = as_f64(unshared_k), as_f64(unshared_v)
    R, BW, Hq, D = q.shape
    Hkv = sk.shape[1]
    G = Hq // Hkv
    scale = scale if scale else 1.0 / np.sqrt(D)
    hist = histories(parent_idx, step)
    out = np.empty((R, BW, Hq, D))
    for r in range(R):
        L = int(prompt_len[r])
        for b in range(BW):
            for h in range(Hq):
                k = h // G
                keys = [sk[r, k, j] for j in range(L)] + [uk[r, k, t, s] for (t, s) in hist[r][b]]
                vals = [sv[r, k, j] for j in range(L)] + [uv[r, k, t, s] for (t, s) in hist[r][b]]
                K = np.stack(keys)
                V = np.stack(vals)
                x = scale * (K @ q[r, b, h])
                w = np.exp(x - x.max())
                out[r, b, h] = (w @ V) / w.sum()
    return out
