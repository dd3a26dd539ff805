"""CPU oracle for staged beam-search decode attention (float64).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library under
``generative_recommendation_beam_xattn_amd/`` and imports nothing from it.

What it computes follows the xGR technical summary (gist.science, paper
2512.11529), section 2.1 "xAttention": a Shared stage over the request's
prompt KV, an Unshared stage over the beam's own generated tokens reached
through per-step parent indices, and an OnlineSoftmax merge of the two.  The
C source ``xattn_oracle.c`` holds the arithmetic and states each reading
taken where the page is silent.  Every function here is pinned by
``tests/test_oracle_pins.py`` against brute force, library attention,
closed forms and invariants.

Arrays are numpy; bf16 tensors are passed as their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "xattn_oracle.c"), os.path.join(_HERE, "beam_topk_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < max(os.path.getmtime(s) for s in _SRCS))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                        "-Wall", "-o", tmp] + _SRCS + ["-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("BW", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("Lmax", ctypes.c_int32),
                ("S", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_double)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.c_void_p
            lib.oracle_ancestors.argtypes = [ctypes.c_int32] * 3 + [P, ctypes.c_int32, P]
            lib.oracle_ancestors.restype = ctypes.c_int
            lib.oracle_attend.argtypes = [P] * 8 + [ctypes.c_int32, ctypes.c_int64, P, P, P]
            lib.oracle_attend.restype = ctypes.c_int
            lib.oracle_stage_partials.argtypes = ([P] * 8 + [ctypes.c_int32, ctypes.c_int64]
                                                  + [P] * 5)
            lib.oracle_stage_partials.restype = ctypes.c_int
            lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int32] + [P] * 6
            lib.oracle_merge.restype = None
            lib.oracle_beam_topk.argtypes = [ctypes.c_int32] * 3 + [P] * 6
            lib.oracle_beam_topk.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("oracle inputs must be float32 or bf16 bit patterns (uint16), got %s" % a.dtype)


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def ancestors(parent_idx: np.ndarray, step: int) -> np.ndarray:
    """anc[r][b][t], t = 0..step: slot of beam b's ancestor at level t."""
    p = _c(parent_idx, np.int32)
    R, S, BW = p.shape
    anc = np.empty((R, BW, step + 1), np.int32)
    rc = _load().oracle_ancestors(R, BW, S, _ptr(p), int(step), _ptr(anc))
    if rc != 0:
        raise ValueError("oracle_ancestors: invalid step or parent index out of range")
    return anc


def _shape_and_arrays(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx,
                      scale):
    q, shared_k, shared_v = _c(q), _c(shared_k), _c(shared_v)
    unshared_k, unshared_v = _c(unshared_k), _c(unshared_v)
    prompt_len = _c(prompt_len, np.int32)
    parent_idx = _c(parent_idx, np.int32)
    R, BW, Hq, D = q.shape
    _, Hkv, Lmax, _ = shared_k.shape
    S = unshared_k.shape[2]
    code = _dtype_code(q)
    for a in (shared_k, shared_v, unshared_k, unshared_v):
        if _dtype_code(a) != code:
            raise TypeError("q, k and v must share one dtype")
    if shared_k.shape != (R, Hkv, Lmax, D) or shared_v.shape != shared_k.shape:
        raise ValueError("shared cache must be [R][Hkv][Lmax][D]")
    if unshared_k.shape != (R, Hkv, S, BW, D) or unshared_v.shape != unshared_k.shape:
        raise ValueError("unshared cache must be [R][Hkv][S][BW][D]")
    if prompt_len.shape != (R,) or parent_idx.shape != (R, S, BW):
        raise ValueError("prompt_len must be [R], parent_idx [R][S][BW]")
    sc = float(scale) if scale else 1.0 / np.sqrt(D)
    shp = _Shape(R, BW, Hq, Hkv, D, Lmax, S, code, sc)
    return shp, (q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx)


def _rows_arg(rows):
    if rows is None:
        return None, 0
    rows = _c(rows, np.int32).reshape(-1, 3)
    return rows, rows.shape[0]


def attend(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
           rows=None, scale=None):
    """Softmax attention over [shared rows 0..L_r-1 ; ancestor tokens 0..step].

    Returns (out, lse): out [R][BW][Hq][D] float64 and lse [R][BW][Hq], or,
    when ``rows`` ([n][3] of (r, b, h)) is given, out [n][D] and lse [n].
    """
    shp, arrs = _shape_and_arrays(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v,
                                  parent_idx, scale)
    rows, n = _rows_arg(rows)
    if rows is None:
        out = np.empty(q.shape, np.float64)
        lse = np.empty(q.shape[:3], np.float64)
    else:
        out = np.empty((n, shp.D), np.float64)
        lse = np.empty((n,), np.float64)
    rc = _load().oracle_attend(ctypes.byref(shp), *[_ptr(a) for a in arrs], int(step), n,
                               _ptr(rows), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attend: invalid arguments, prompt length or parent index")
    return out, lse


def stage_partials(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v, parent_idx, step,
                   rows=None, scale=None):
    """Per-stage (m, l, o) of the Shared and Unshared stages, each on its own.

    Returns dict with shared_ml, shared_o, unshared_ml, unshared_o; *_ml has a
    trailing axis (m, l) and *_o a trailing axis D, leading axes as in attend().
    """
    shp, arrs = _shape_and_arrays(q, shared_k, shared_v, prompt_len, unshared_k, unshared_v,
                                  parent_idx, scale)
    rows, n = _rows_arg(rows)
    lead = q.shape[:3] if rows is None else (n,)
    res = {"shared_ml": np.empty(lead + (2,), np.float64),
           "shared_o": np.empty(lead + (shp.D,), np.float64),
           "unshared_ml": np.empty(lead + (2,), np.float64),
           "unshared_o": np.empty(lead + (shp.D,), np.float64)}
    rc = _load().oracle_stage_partials(ctypes.byref(shp), *[_ptr(a) for a in arrs], int(step), n,
                                       _ptr(rows), _ptr(res["shared_ml"]), _ptr(res["shared_o"]),
                                       _ptr(res["unshared_ml"]), _ptr(res["unshared_o"]))
    if rc != 0:
        raise ValueError("oracle_stage_partials: invalid arguments")
    return res


def merge(ml_a, o_a, ml_b, o_b):
    """OnlineSoftmax combine of two partials; returns (out, lse)."""
    ml_a = _c(ml_a, np.float64)
    o_a = _c(o_a, np.float64)
    ml_b = _c(ml_b, np.float64)
    o_b = _c(o_b, np.float64)
    D = o_a.shape[-1]
    n = o_a.size // D
    out = np.empty(o_a.shape, np.float64)
    lse = np.empty(o_a.shape[:-1], np.float64)
    _load().oracle_merge(n, D, _ptr(ml_a), _ptr(o_a), _ptr(ml_b), _ptr(o_b), _ptr(out), _ptr(lse))
    return out, lse


def reorder_unshared(cache, parent, n_levels: int):
    """In-place reorder of the Unshared cache after beam selection, as a copy.

    xGR summary, section 2.1 ("in-place updates"): instead of following
    parent chains, the generated-token rows are moved so that slot b holds
    beam b's own history.  After a step's selection, with parent[r][b] the
    slot the new beam b descends from, every row (level t < n_levels, slot
    b) takes the old row (t, parent[r][b]), for every KV head.  cache is
    [R][Hkv][S][BW][D] (any dtype), parent [R][BW]; returns the new cache.
    """
    cache = np.asarray(cache)
    parent = np.asarray(parent, np.int64)
    R, Hkv, S, BW, D = cache.shape
    if parent.shape != (R, BW) or not 0 <= n_levels <= S:
        raise ValueError("parent must be [R][BW] and 0 <= n_levels <= S")
    if parent.size and (parent.min() < 0 or parent.max() >= BW):
        raise ValueError("parent index out of range")
    out = cache.copy()
    for r in range(R):
        for t in range(n_levels):
            for b in range(BW):
                out[r, :, t, b, :] = cache[r, :, t, parent[r, b], :]
    return out


def valid_next_tokens(items, prefix) -> np.ndarray:
    """Tokens that may follow `prefix` on a valid path (xGR summary, section
    2.2: xBeam's valid-path constraint, masks generated from a pre-built
    vocabulary of valid items).  Brute force over the item list: token j is
    valid after prefix p (length d) iff some item starts with p and has j at
    position d.  items [N][L] int; prefix a sequence of d < L tokens, or
    None for a dead beam (no valid continuation).  Returns sorted tokens."""
    items = np.asarray(items)
    if prefix is None:
        return np.zeros(0, np.int64)
    d = len(prefix)
    if not 0 <= d < items.shape[1]:
        raise ValueError("prefix length must be in [0, L)")
    hit = np.all(items[:, :d] == np.asarray(prefix, items.dtype)[None, :], axis=1)
    return np.unique(items[hit, d]).astype(np.int64)


def apply_valid_mask(items, prefixes, logits):
    """Masked logits: every token that is not a valid continuation of its
    beam's prefix becomes -inf, the others keep their value.  prefixes is a
    list (one per row of logits [n][V]) of token sequences or None."""
    logits = np.asarray(logits, np.float32)
    out = np.full_like(logits, -np.inf)
    for i, p in enumerate(prefixes):
        ok = valid_next_tokens(items, p)
        out[i, ok] = logits[i, ok]
    return out


def beam_topk(cum, logp, token):
    """Beam selection of one decode step (xGR summary, section 2.2 "xBeam").

    cum [R][BW] float32, logp [R][BW][V] float32 (rows sorted descending),
    token [R][BW][V] int32.  Every candidate (b, j) scores the float32 sum
    cum[b] + logp[b][j]; the BW best under (score desc, parent asc, token asc)
    are returned in that order as (score [R][BW] float32, parent [R][BW]
    int32, token [R][BW] int32).
    """
    cum = _c(cum, np.float32)
    logp = _c(logp, np.float32)
    token = _c(token, np.int32)
    R, BW, V = logp.shape
    if cum.shape != (R, BW) or token.shape != (R, BW, V):
        raise ValueError("cum must be [R][BW] and token [R][BW][V] for logp [R][BW][V]")
    score = np.empty((R, BW), np.float32)
    parent = np.empty((R, BW), np.int32)
    new_token = np.empty((R, BW), np.int32)
    rc = _load().oracle_beam_topk(R, BW, V, _ptr(cum), _ptr(logp), _ptr(token), _ptr(score),
                                  _ptr(parent), _ptr(new_token))
    if rc != 0:
        raise ValueError("oracle_beam_topk: empty shape or NaN score")
    return score, parent, new_token


def omp_threads() -> int:
    """Threads the OpenMP runtime of the oracle will use (OMP_NUM_THREADS or cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))
