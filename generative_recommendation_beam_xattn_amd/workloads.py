"""Seeded synthetic decode-attention inputs.

This module only draws random inputs; it holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

The workload shapes follow the xGR technical summary (gist.science, paper
2512.11529): section 1 describes generative recommendation as long
user-history prompts, short fixed-length outputs and wide beams (candidate
pools of 128x128 and 512x512), and section 4 sweeps the beam width from 128
to 512.  The prefix-homogeneity sweep follows the Feather summary
(gist.science, paper 2605.06046), "Risultati": request groups that share a
long prefix.  The pages measure on Amazon Review, JD Trace, L-Eval and
LongBench; none of those is used here -- these seeded synthetic arrays of the
same shape stand in for them.

Recipe (fixed so every consumer sees identical bytes):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * values: standard normal drawn as float32, rounded to bfloat16 by
    round-to-nearest-even where the workload is bf16 (stored as uint16 bit
    patterns);
  * draw order: prompt_len, q (all decode steps), shared_k, shared_v,
    unshared_k, unshared_v, parent_idx;
  * every level of the unshared cache is filled (the caller writes the
    current level before each call; levels above the step are never read).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 24  # elements per draw, bounds the float32 temporaries


@dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    R: int
    BW: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    S: int
    steps: list                # decode steps (levels) one pass runs, in order
    prompt_len: np.ndarray     # int32 [R]
    q: np.ndarray              # [len(steps)][R][BW][Hq][D]
    shared_k: np.ndarray       # [R][Hkv][Lmax][D]
    shared_v: np.ndarray
    unshared_k: np.ndarray     # [R][Hkv][S][BW][D]
    unshared_v: np.ndarray
    parent_idx: np.ndarray     # int32 [R][S][BW]
    meta: dict = field(default_factory=dict)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Standard normal values of ``shape`` drawn in chunks (same stream as one draw)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32 if dtype == "f32" else np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else to_bf16_bits(x)
    return out.reshape(shape)


# The five workloads: tiny plumbing case, GR serving shape, large batch,
# wide-beam stress, prefix-homogeneity sweep (G sequences per prefix group).
CONFIGS = {
    1: dict(name="tiny", seed=1, R=1, L=(128, 128), BW=4, steps=[0, 1, 2], Hq=4, Hkv=4, D=64,
            dtype="f32", parents="uniform", S=3),
    2: dict(name="gr_serving", seed=2, R=16, L=(512, 1024), BW=128, steps=[0, 1, 2], Hq=16,
            Hkv=4, D=128, dtype="bf16", parents="uniform", S=3),
    3: dict(name="large_batch", seed=3, R=64, L=(2048, 2048), BW=256, steps=[0, 1, 2], Hq=32,
            Hkv=8, D=128, dtype="bf16", parents="skewed", S=3),
    4: dict(name="wide_beam", seed=4, R=8, L=(4096, 4096), BW=512, steps=[0, 1, 2, 3], Hq=32,
            Hkv=8, D=128, dtype="bf16", parents="uniform", S=4),
    5: dict(name="prefix_sweep", seed=5, R=None, L=(3584, 3584), BW=None, steps=[511], Hq=32,
            Hkv=8, D=128, dtype="bf16", parents="identity", S=512),
}
PREFIX_GROUPS = (1, 8, 32, 256)
PREFIX_SEQUENCES = 256


def _parents(rng, kind: str, R: int, S: int, BW: int) -> np.ndarray:
    if kind == "uniform":
        return rng.integers(0, BW, size=(R, S, BW), dtype=np.int32)
    if kind == "identity":
        return np.broadcast_to(np.arange(BW, dtype=np.int32), (R, S, BW)).copy()
    if kind == "skewed":
        # Per level, a random half of the beams draw their parent from the
        # 16 best-ranked slots (slots 0..15); the other half from all slots.
        p = np.empty((R, S, BW), np.int32)
        top = min(16, BW)
        for r in range(R):
            for t in range(S):
                chosen = rng.permutation(BW)[: BW // 2]
                row = rng.integers(0, BW, size=BW, dtype=np.int32)
                row[chosen] = rng.integers(0, top, size=chosen.size, dtype=np.int32)
                p[r, t] = row
        return p
    raise ValueError(kind)


def make(config: int, G: int | None = None, *, R: int | None = None) -> Workload:
    """Build workload ``config`` (1..5).  Config 5 needs the group size G.

    ``R`` optionally truncates the request count (draws stay a prefix of the
    full stream only for the prompt lengths; use it for smaller variants).
    """
    c = dict(CONFIGS[config])
    if config == 5:
        if G not in PREFIX_GROUPS:
            raise ValueError("config 5 needs G in %s" % (PREFIX_GROUPS,))
        c["R"] = PREFIX_SEQUENCES // G
        c["BW"] = G
        c["name"] = "prefix_sweep_G%d" % G
    if R is not None:
        c["R"] = R
    return custom(name=c["name"], seed=c["seed"], R=c["R"], L=c["L"], BW=c["BW"],
                  steps=c["steps"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"],
                  parents=c["parents"], S=c["S"], Lmax=c["L"][1],
                  meta={"config": config, "G": G})


def custom(*, name="custom", seed=0, R, L, BW, steps, Hq, Hkv, D, dtype="bf16",
           parents="uniform", S=None, Lmax=None, meta=None) -> Workload:
    """Any shape.  ``L`` is an int, a tuple (lo, hi) drawn uniformly (inclusive),
    or a list / array of R explicit lengths."""
    rng = np.random.default_rng(seed)
    S = S if S is not None else max(steps) + 1
    if isinstance(L, tuple):
        lo, hi = L
        prompt_len = (np.full(R, lo, np.int32) if lo == hi
                      else rng.integers(lo, hi + 1, size=R, dtype=np.int32))
    elif isinstance(L, (list, np.ndarray)):
        prompt_len = np.asarray(L, np.int32)
        if prompt_len.shape != (R,):
            raise ValueError("explicit prompt lengths must have R entries")
    else:
        prompt_len = np.full(R, int(L), np.int32)
    Lmax = int(Lmax if Lmax is not None else max(1, int(prompt_len.max())))
    q = normal(rng, (len(steps), R, BW, Hq, D), dtype)
    shared_k = normal(rng, (R, Hkv, Lmax, D), dtype)
    shared_v = normal(rng, (R, Hkv, Lmax, D), dtype)
    unshared_k = normal(rng, (R, Hkv, S, BW, D), dtype)
    unshared_v = normal(rng, (R, Hkv, S, BW, D), dtype)
    parent_idx = _parents(rng, parents, R, S, BW)
    return Workload(name=name, dtype=dtype, R=R, BW=BW, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, S=S,
                    steps=list(steps), prompt_len=prompt_len, q=q, shared_k=shared_k,
                    shared_v=shared_v, unshared_k=unshared_k, unshared_v=unshared_v,
                    parent_idx=parent_idx, meta=dict(meta or {}, seed=seed, parents=parents))


# --- beam-selection inputs --------------------------------------------------
#
# One decode step's candidate pool for beam selection (xGR summary, section
# 2.2 "xBeam"; pool sizes 128x128 and 512x512 from its section 1): every beam
# of a request proposes its V best next tokens, sorted by log-probability.
# Recipe (generator ``numpy.random.default_rng(seed)``, draw order cum,
# logp, token):
#   * cum [R][BW]: cumulative beam scores, -3 + N(0, 1) as float32;
#   * logp [R][BW][V]: per row, V draws of 2 * N(0, 1) as float32, sorted
#     descending, minus the row maximum and ln(VOCAB) so they look like
#     log-probabilities (<= -ln VOCAB);
#   * token [R][BW][V]: per row, V distinct ids from a vocabulary of VOCAB
#     (a random permutation's first V entries).
# Variants for edge cases: "ties" rounds cum and logp to multiples of 1/4
# (many equal scores, across and within rows, in random token order);
# "identical" gives every beam of a request the same cum, logp and token
# rows (the first step of a search, when all beams hold the same prefix);
# ``masked_frac`` sets that fraction of each row's tail to -inf, as an
# item-validity mask does to tokens that lead to no valid item.
BEAM_VOCAB = 8192
BEAM_POOLS = {"gr_serving": dict(R=16, BW=128, V=128), "wide_beam": dict(R=8, BW=512, V=512)}


@dataclass
class BeamPool:
    cum: np.ndarray      # float32 [R][BW]
    logp: np.ndarray     # float32 [R][BW][V], rows non-increasing
    token: np.ndarray    # int32 [R][BW][V]

    @property
    def shape(self):
        return self.logp.shape


def beam_pool(seed: int, R: int, BW: int, V: int, kind: str = "normal",
              masked_frac: float = 0.0, vocab: int = BEAM_VOCAB) -> BeamPool:
    if V > vocab:
        raise ValueError("V must not exceed the vocabulary")
    rng = np.random.default_rng(seed)
    cum = (np.float32(-3.0) + rng.standard_normal((R, BW), dtype=np.float32)).astype(np.float32)
    x = np.float32(2.0) * rng.standard_normal((R, BW, V), dtype=np.float32)
    x = -np.sort(-x, axis=-1)
    logp = (x - x[..., :1] - np.float32(np.log(vocab))).astype(np.float32)
    token = np.empty((R, BW, V), np.int32)
    for r in range(R):
        for b in range(BW):
            token[r, b] = rng.permutation(vocab)[:V]
    if kind == "ties":
        cum = (np.round(cum * 4) / 4).astype(np.float32)
        logp = (np.round(logp * 4) / 4).astype(np.float32)
    elif kind == "identical":
        cum = np.repeat(cum[:, :1], BW, axis=1)
        logp = np.repeat(logp[:, :1], BW, axis=1)
        token = np.repeat(token[:, :1], BW, axis=1)
    elif kind != "normal":
        raise ValueError(kind)
    if masked_frac > 0:
        n = int(round(masked_frac * V))
        if n:
            logp[..., V - n:] = -np.inf
    return BeamPool(cum=np.ascontiguousarray(cum), logp=np.ascontiguousarray(logp),
                    token=np.ascontiguousarray(token))


# --- valid-item vocabularies ------------------------------------------------
#
# Items are fixed-length token paths (xGR summary, section 1: items are
# identified by token sequences, most sequences map to no item; section 2.2:
# a pre-built vocabulary of valid items drives the masks).  Recipe (generator
# ``numpy.random.default_rng(seed)``): the first token of an item follows a
# Zipf-like law over the vocabulary (rank r drawn with weight 1 / (r + 1),
# ranks mapped to ids by a random permutation), every later token is uniform
# over the vocabulary; duplicate items are kept (a vocabulary may list an
# item twice).  The full-size vocabulary is 2^20 items of 3 tokens over 8192
# ids, matching the 3 decode steps of the serving workload.
VALID_ITEMS_FULL = dict(n_items=1 << 20, levels=3, vocab=8192)


def valid_items(seed: int, n_items: int, levels: int, vocab: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, vocab + 1)
    first = rng.permutation(vocab)[rng.choice(vocab, size=n_items, p=w / w.sum())]
    rest = rng.integers(0, vocab, size=(n_items, levels - 1))
    return np.concatenate([first[:, None], rest], axis=1).astype(np.int32)
