"""Pins of the Unshared-cache reorder oracle (oracle.reorder_unshared).

The reorder moves generated-token rows so that slot b holds beam b's own
history (xGR summary, section 2.1, in-place updates).  Checked against
  * beam histories simulated forward by copying (tests/brute.py), which
    follow no parent chain backwards;
  * the oracle's ancestor chains (themselves pinned by that simulation);
  * attention: over the reordered cache with identity parents it equals, bit
    for bit in float64, attention over the original cache with the chains;
  * identity and constant parent rows.
"""
import numpy as np
import pytest

import oracle
from generative_recommendation_beam_xattn_amd import workloads as W
from tests import brute


def tagged_cache(R, Hkv, S, BW, D):
    # row (r, k, t, b) carries its own coordinates, so every move is visible
    c = np.zeros((R, Hkv, S, BW, D), np.float32)
    r, k, t, b = np.meshgrid(np.arange(R), np.arange(Hkv), np.arange(S), np.arange(BW),
                             indexing="ij")
    c[..., 0] = r
    c[..., 1] = k
    c[..., 2] = t
    c[..., 3] = b
    return c


def reorder_pipeline(cache, parent_idx, step):
    # what a caller does: after the selection that yields parent_idx[:, s, :],
    # reorder levels 0..s-1, then level s is written in place (here: kept)
    out = cache
    for s in range(1, step + 1):
        out = oracle.reorder_unshared(out, parent_idx[:, s, :], s)
    return out


@pytest.mark.parametrize("BW,S,step", [(4, 4, 3), (8, 6, 5), (5, 3, 1), (16, 5, 4)])
def test_reorder_matches_forward_histories(BW, S, step):
    R, Hkv, D = 3, 2, 4
    rng = np.random.default_rng(BW + 10 * S)
    p = rng.integers(0, BW, size=(R, S, BW), dtype=np.int32)
    got = reorder_pipeline(tagged_cache(R, Hkv, S, BW, D), p, step)
    hist = brute.histories(p, step)
    for r in range(R):
        for b in range(BW):
            for (t, slot) in hist[r][b]:
                for k in range(Hkv):
                    assert tuple(got[r, k, t, b, :4]) == (r, k, t, slot)


def test_reorder_matches_chains():
    R, Hkv, S, BW, D = 2, 3, 7, 9, 4
    rng = np.random.default_rng(3)
    p = rng.integers(0, BW, size=(R, S, BW), dtype=np.int32)
    step = S - 1
    got = reorder_pipeline(tagged_cache(R, Hkv, S, BW, D), p, step)
    anc = oracle.ancestors(p, step)
    assert (got[:, :, : step + 1, :, 3] == anc.transpose(0, 2, 1)[:, None]).all()


def test_identity_and_constant_rows():
    R, Hkv, S, BW, D = 2, 2, 4, 6, 4
    c = tagged_cache(R, Hkv, S, BW, D)
    ident = np.broadcast_to(np.arange(BW, dtype=np.int32), (R, BW))
    assert np.array_equal(oracle.reorder_unshared(c, ident, S), c)
    const = np.full((R, BW), 4, np.int32)
    got = oracle.reorder_unshared(c, const, 2)
    assert (got[:, :, :2, :, 3] == 4).all()
    assert np.array_equal(got[:, :, 2:], c[:, :, 2:])   # levels past n_levels untouched


def test_rejects_bad_parents():
    c = tagged_cache(1, 1, 2, 3, 4)
    with pytest.raises(ValueError):
        oracle.reorder_unshared(c, np.array([[0, 3, 1]]), 2)
    with pytest.raises(ValueError):
        oracle.reorder_unshared(c, np.array([[0, 1, 1]]), 3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_over_reordered_cache_equals_chains(dtype):
    # the reorder changes where rows live, not what a beam attends to
    w = W.custom(name="reorder", seed=11, R=2, L=[70, 33], BW=6, steps=[3], Hq=4, Hkv=2, D=64,
                 dtype=dtype, S=4)
    step = 3
    chains, _ = oracle.attend(w.q[0], w.shared_k, w.shared_v, w.prompt_len, w.unshared_k,
                              w.unshared_v, w.parent_idx, step)
    uk = reorder_pipeline(w.unshared_k, w.parent_idx, step)
    uv = reorder_pipeline(w.unshared_v, w.parent_idx, step)
    ident = np.broadcast_to(np.arange(w.BW, dtype=np.int32), w.parent_idx.shape).copy()
    moved, _ = oracle.attend(w.q[0], w.shared_k, w.shared_v, w.prompt_len, uk, uv, ident, step)
    assert np.array_equal(chains, moved)
