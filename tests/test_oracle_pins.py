"""Pins for the CPU oracle (no GPU).

The reference pages print no worked example and no formula for the staged
attention, so the oracle is pinned to things other than itself:
  * brute force: beam histories simulated forward by copying, full sequences
    materialised, numpy softmax attention (tests/brute.py);
  * a library special case: with one beam the path is ordinary
    single-sequence attention, checked against torch's
    scaled_dot_product_attention in float64;
  * closed forms: constant values, a zero query, a single token, hand-built
    scores with known softmax weights, distinct per-head values for the GQA
    head mapping;
  * invariants: merge associativity over any split of the shared range, a
    common shift of every key, relabelling of the current beam slots.
Each is chosen so that a plausible mistake (a dropped level, an off-by-one
in the parent chain, the wrong KV head, a wrong scale, reading past the
prompt length) fails at least one of them.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from generative_recommendation_beam_xattn_amd import workloads as W
from tests import brute

TOL = 1e-12


def _wl(seed=0, R=2, BW=3, Hq=4, Hkv=2, D=16, L=(0, 20), steps=(2,), dtype="f32", S=None,
        parents="uniform", Lmax=None):
    return W.custom(seed=seed, R=R, L=L, BW=BW, steps=list(steps), Hq=Hq, Hkv=Hkv, D=D,
                    dtype=dtype, S=S, parents=parents, Lmax=Lmax)


def _args(w, i=0):
    return (w.q[i], w.shared_k, w.shared_v, w.prompt_len, w.unshared_k, w.unshared_v,
            w.parent_idx, w.steps[i])


# ---------------------------------------------------------------- ancestors

@pytest.mark.parametrize("BW,S,step", [(1, 1, 0), (4, 3, 2), (7, 6, 5), (16, 9, 8), (3, 5, 1)])
def test_ancestors_match_forward_simulation(BW, S, step):
    rng = np.random.default_rng(BW * 100 + S)
    p = rng.integers(0, BW, size=(3, S, BW), dtype=np.int32)
    anc = oracle.ancestors(p, step)
    hist = brute.histories(p, step)
    for r in range(3):
        for b in range(BW):
            assert [s for (_, s) in hist[r][b]] == list(anc[r, b])
            assert [t for (t, _) in hist[r][b]] == list(range(step + 1))


def test_ancestors_identity_and_constant_row():
    BW, S = 8, 6
    ident = np.broadcast_to(np.arange(BW, dtype=np.int32), (2, S, BW)).copy()
    anc = oracle.ancestors(ident, S - 1)
    assert (anc == np.arange(BW)[None, :, None]).all()
    # a constant parent row at level 3: every beam shares its level-2 ancestor
    # and everything below it
    rng = np.random.default_rng(7)
    p = rng.integers(0, BW, size=(1, S, BW), dtype=np.int32)
    p[0, 3, :] = 5
    anc = oracle.ancestors(p, 4)
    assert (anc[0, :, 2] == 5).all()
    assert (anc[0, :, :3] == anc[0, :1, :3]).all()


def test_ancestors_row_zero_is_ignored():
    p = np.zeros((1, 3, 4), np.int32)
    p[0, 0, :] = 99  # out of range but never read
    p[0, 1:, :] = [[1, 0, 3, 2], [2, 2, 0, 1]]
    anc = oracle.ancestors(p, 2)
    # beam 0: level-2 slot 0 -> level-1 slot p[2][0] = 2 -> level-0 slot p[1][2] = 3
    assert anc[0, 0].tolist() == [3, 2, 0]
    hist = brute.histories(p, 2)
    assert [s for (_, s) in hist[0][0]] == anc[0, 0].tolist()


def test_ancestors_reject_out_of_range():
    p = np.zeros((1, 3, 4), np.int32)
    p[0, 2, 1] = 4
    with pytest.raises(ValueError):
        oracle.ancestors(p, 2)


# --------------------------------------------------------------- brute force

CASES = [
    dict(R=1, BW=1, Hq=1, Hkv=1, D=8, L=(5, 5), steps=(0,)),
    dict(R=2, BW=3, Hq=4, Hkv=2, D=16, L=(0, 20), steps=(2,)),
    dict(R=3, BW=5, Hq=6, Hkv=3, D=8, L=[0, 1, 33], steps=(3,), S=5),
    dict(R=1, BW=4, Hq=4, Hkv=4, D=64, L=(128, 128), steps=(2,)),          # tiny config shape
    dict(R=2, BW=6, Hq=8, Hkv=2, D=16, L=(10, 40), steps=(4,), dtype="bf16"),
    dict(R=2, BW=2, Hq=2, Hkv=1, D=8, L=(3, 9), steps=(1,), parents="identity"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attend_matches_brute_force(case):
    w = _wl(seed=case, **CASES[case])
    out, lse = oracle.attend(*_args(w))
    ref = brute.attend(*_args(w))
    assert np.max(np.abs(out - ref)) <= TOL
    assert np.isfinite(lse).all()


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(R=st.integers(1, 3), BW=st.integers(1, 6), step=st.integers(0, 4), L=st.integers(0, 40),
       G=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 2), D=st.sampled_from([8, 16]),
       dtype=st.sampled_from(["f32", "bf16"]), seed=st.integers(0, 2**16))
def test_attend_brute_force_random(R, BW, step, L, G, Hkv, D, dtype, seed):
    w = _wl(seed=seed, R=R, BW=BW, Hq=G * Hkv, Hkv=Hkv, D=D, L=(0, L), steps=(step,),
            dtype=dtype, S=step + 2)
    out, _ = oracle.attend(*_args(w))
    ref = brute.attend(*_args(w))
    assert np.max(np.abs(out - ref)) <= TOL


def test_attend_never_reads_past_prompt_or_step():
    w = _wl(seed=3, R=2, BW=4, Hq=4, Hkv=2, D=16, L=[7, 0], steps=(1,), S=4, Lmax=12)
    clean = brute.attend(*_args(w))
    # poison shared rows >= L_r and unshared levels > step with NaN
    for a in (w.shared_k, w.shared_v):
        for r, L in enumerate(w.prompt_len):
            a[r, :, L:] = np.nan
    for a in (w.unshared_k, w.unshared_v):
        a[:, :, 2:] = np.nan
    w.parent_idx[:, 0] = -1  # row 0 is never read either
    w.parent_idx[:, 2:] = -1
    out, _ = oracle.attend(*_args(w))
    assert np.isfinite(out).all()
    assert np.max(np.abs(out - clean)) <= TOL


def test_rows_subset_matches_full():
    w = _wl(seed=11, R=3, BW=5, Hq=4, Hkv=2, D=16, L=(0, 30), steps=(3,))
    full, lse_full = oracle.attend(*_args(w))
    rows = np.array([[0, 0, 0], [2, 4, 3], [1, 2, 1], [2, 0, 2]], np.int32)
    sub, lse_sub = oracle.attend(*_args(w), rows=rows)
    for i, (r, b, h) in enumerate(rows):
        assert np.array_equal(sub[i], full[r, b, h])
        assert lse_sub[i] == lse_full[r, b, h]


# ----------------------------------------------------------- library special case

@pytest.mark.parametrize("Hq,Hkv,D,L,step", [(4, 4, 64, 128, 2), (16, 4, 128, 300, 3),
                                             (8, 2, 32, 0, 1)])
def test_single_beam_is_standard_attention(Hq, Hkv, D, L, step):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    w = _wl(seed=5, R=2, BW=1, Hq=Hq, Hkv=Hkv, D=D, L=(L, L), steps=(step,), S=step + 1,
            Lmax=max(L, 1))
    out, _ = oracle.attend(*_args(w))
    G = Hq // Hkv
    for r in range(w.R):
        Lr = int(w.prompt_len[r])
        K = np.concatenate([w.shared_k[r, :, :Lr], w.unshared_k[r, :, : step + 1, 0]], axis=1)
        V = np.concatenate([w.shared_v[r, :, :Lr], w.unshared_v[r, :, : step + 1, 0]], axis=1)
        Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(G, dim=0)
        Qt = torch.from_numpy(w.q[0][r, 0].astype(np.float64))[:, None, :]
        ref = F.scaled_dot_product_attention(Qt, Kt, Vt)[:, 0, :].numpy()
        assert np.max(np.abs(out[r, 0] - ref)) <= TOL


# ------------------------------------------------------------------ closed forms

def test_constant_values_give_the_constant():
    w = _wl(seed=21, R=2, BW=5, Hq=8, Hkv=2, D=16, L=(0, 50), steps=(3,), S=4)
    c = np.float32(0.625)
    for a in (w.shared_v, w.unshared_v):
        a[...] = c
    out, _ = oracle.attend(*_args(w))
    assert np.max(np.abs(out - c)) <= TOL


def test_zero_query_gives_mean_of_attended_values():
    w = _wl(seed=22, R=2, BW=4, Hq=4, Hkv=2, D=16, L=(3, 25), steps=(2,))
    w.q[...] = 0
    out, lse = oracle.attend(*_args(w))
    hist = brute.histories(w.parent_idx, 2)
    sv, uv = brute.as_f64(w.shared_v), brute.as_f64(w.unshared_v)
    for r in range(w.R):
        L = int(w.prompt_len[r])
        for b in range(w.BW):
            for h in range(w.Hq):
                k = h // 2
                rows = [sv[r, k, j] for j in range(L)] + [uv[r, k, t, s] for t, s in hist[r][b]]
                assert np.max(np.abs(out[r, b, h] - np.mean(rows, axis=0))) <= TOL
                assert abs(lse[r, b, h] - np.log(L + 3)) <= TOL


def test_single_token_is_its_value_exactly():
    w = _wl(seed=23, R=2, BW=3, Hq=4, Hkv=2, D=16, L=(0, 0), steps=(0,), S=2, dtype="bf16")
    out, lse = oracle.attend(*_args(w))
    uv = brute.as_f64(w.unshared_v)
    for r, b, h in itertools.product(range(2), range(3), range(4)):
        assert np.array_equal(out[r, b, h], uv[r, h // 2, 0, b])
    q = brute.as_f64(w.q[0])
    uk = brute.as_f64(w.unshared_k)
    for r, b, h in itertools.product(range(2), range(3), range(4)):
        assert abs(lse[r, b, h] - q[r, b, h] @ uk[r, h // 2, 0, b] / 4.0) <= TOL


def test_hand_built_scores_give_known_weights():
    """D = 4 (scale 1/2), query (2,0,0,0): a key's score is its first entry.

    The beam in slot 1 at level 1 descends from slot 0 at level 0.  Its
    attended keys are: shared row 0 (score 0), level-0 slot 0 (score ln 2)
    and level-1 slot 1 (score ln 3), so the weights are 1/6, 2/6, 3/6 and
    the output is (1/6, 2/6, 3/6, 0) for values e1, e2, e3.  Every other row
    is a decoy with a large score and a distinct value: reading the wrong
    ancestor, level, shared row or KV head changes the result.
    """
    R, BW, Hq, Hkv, D, Lmax, S = 1, 2, 2, 2, 4, 3, 2
    q = np.zeros((R, BW, Hq, D), np.float32)
    q[0, :, :, 0] = 2.0
    sk = np.zeros((R, Hkv, Lmax, D), np.float32)
    sv = np.zeros((R, Hkv, Lmax, D), np.float32)
    uk = np.zeros((R, Hkv, S, BW, D), np.float32)
    uv = np.zeros((R, Hkv, S, BW, D), np.float32)
    for k in range(Hkv):
        sk[0, k, 0, 0] = 0.0
        sv[0, k, 0] = [1, 0, 0, 0]
        sk[0, k, 1:, 0] = 9.0          # beyond prompt_len: must not be read
        sv[0, k, 1:, 3] = 100.0
        uk[0, k, 0, 0, 0] = np.log(2.0)
        uv[0, k, 0, 0] = [0, 1, 0, 0]
        uk[0, k, 0, 1, 0] = 8.0        # level-0 slot 1: not an ancestor of beam 1
        uv[0, k, 0, 1, 3] = 50.0
        uk[0, k, 1, 1, 0] = np.log(3.0)
        uv[0, k, 1, 1] = [0, 0, 1, 0]
        uk[0, k, 1, 0, 0] = 7.0        # level-1 slot 0 belongs to beam 0 only
        uv[0, k, 1, 0, 3] = 25.0
    # KV head 1 gets its own decoy in an otherwise unused column; head 1 of
    # q reads KV head 1, head 0 reads KV head 0
    sv[0, 1, 0, 3] = 0.0
    prompt_len = np.array([1], np.int32)
    parent = np.zeros((R, S, BW), np.int32)
    parent[0, 1] = [1, 0]              # level1 slot0 <- slot1, level1 slot1 <- slot0
    out, lse = oracle.attend(q, sk, sv, prompt_len, uk, uv, parent, 1)
    expect = np.array([1 / 6, 2 / 6, 3 / 6, 0])
    for h in range(Hq):
        assert np.max(np.abs(out[0, 1, h] - expect)) <= 1e-7  # ln2, ln3 rounded to fp32
        assert abs(lse[0, 1, h] - np.log(6.0)) <= 1e-7
    # beam 0: shared row 0 (score 0), level-0 slot 1 (score 8), level-1 slot 0 (score 7)
    z = 1 + np.exp(8.0) + np.exp(7.0)
    expect0 = np.array([1 / z, 0, 0, (50 * np.exp(8.0) + 25 * np.exp(7.0)) / z])
    for h in range(Hq):
        assert np.max(np.abs(out[0, 0, h] - expect0)) <= 1e-12


def test_gqa_groups_are_contiguous():
    """Query head h reads KV head h // (Hq/Hkv): give each KV head a constant value."""
    w = _wl(seed=24, R=1, BW=2, Hq=8, Hkv=4, D=8, L=(6, 6), steps=(1,))
    for k in range(4):
        w.shared_v[:, k] = k + 1
        w.unshared_v[:, k] = k + 1
    out, _ = oracle.attend(*_args(w))
    for h in range(8):
        assert np.max(np.abs(out[0, :, h] - (h // 2 + 1))) <= TOL


# ------------------------------------------------------------------- invariants

def _partials_to_ml_o(ml, o):
    return ml.reshape(-1, 2), o.reshape(-1, o.shape[-1])


def test_stage_partials_merge_to_the_definition():
    w = _wl(seed=31, R=3, BW=4, Hq=4, Hkv=2, D=16, L=[0, 5, 40], steps=(3,))
    p = oracle.stage_partials(*_args(w))
    out, lse = oracle.merge(p["shared_ml"], p["shared_o"], p["unshared_ml"], p["unshared_o"])
    ref, ref_lse = oracle.attend(*_args(w))
    assert np.max(np.abs(out - ref)) <= TOL
    assert np.max(np.abs(lse - ref_lse)) <= TOL
    # the empty prompt gives an empty shared partial
    assert np.all(p["shared_ml"][0, ..., 1] == 0) and np.all(np.isneginf(p["shared_ml"][0, ..., 0]))
    assert np.all(p["shared_o"][0] == 0)
    # merging in the other order gives the same answer
    out2, _ = oracle.merge(p["unshared_ml"], p["unshared_o"], p["shared_ml"], p["shared_o"])
    assert np.max(np.abs(out2 - ref)) <= TOL


@pytest.mark.parametrize("cuts", [[0, 7, 7, 19, 64], [0, 64], [0, 1, 2, 3, 64], [0, 32, 64]])
def test_merge_is_associative_over_any_split_of_the_prompt(cuts):
    w = _wl(seed=32, R=2, BW=3, Hq=4, Hkv=2, D=16, L=[64, 23], steps=(2,), Lmax=64)
    ref, ref_lse = oracle.attend(*_args(w))
    q, sk, sv, pl, uk, uv, par, s = _args(w)
    parts = []
    first = oracle.stage_partials(*_args(w))
    parts.append((first["unshared_ml"], first["unshared_o"]))
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        sub_len = np.clip(pl - lo, 0, hi - lo).astype(np.int32)
        p = oracle.stage_partials(q, np.ascontiguousarray(sk[:, :, lo:hi]) if hi > lo else sk[:, :, :1],
                                  np.ascontiguousarray(sv[:, :, lo:hi]) if hi > lo else sv[:, :, :1],
                                  sub_len if hi > lo else np.zeros_like(pl), uk, uv, par, s)
        parts.append((p["shared_ml"], p["shared_o"]))
    for order in (range(len(parts)), reversed(range(len(parts)))):
        order = list(order)
        ml, o = parts[order[0]]
        for i in order[1:]:
            o, lse = oracle.merge(ml, o, *parts[i])
            ml = np.stack([lse, np.ones_like(lse)], axis=-1)
        assert np.max(np.abs(o - ref)) <= TOL
        assert np.max(np.abs(ml[..., 0] - ref_lse)) <= TOL


def test_common_key_shift_leaves_output_unchanged():
    # keys on a 2^-10 grid and integer shifts keep K + delta exact in float32
    w = _wl(seed=33, R=2, BW=4, Hq=4, Hkv=2, D=16, L=(5, 30), steps=(2,))
    for a in (w.shared_k, w.unshared_k):
        a[...] = np.round(a * 1024) / 1024
    base, _ = oracle.attend(*_args(w))
    rng = np.random.default_rng(0)
    delta = rng.integers(-3, 4, size=(w.Hkv, w.D)).astype(np.float32)
    w.shared_k += delta[None, :, None, :]
    w.unshared_k += delta[None, :, None, None, :]
    shifted, _ = oracle.attend(*_args(w))
    assert np.max(np.abs(shifted - base)) <= 1e-10


def test_relabelling_current_slots_permutes_the_output():
    w = _wl(seed=34, R=2, BW=6, Hq=4, Hkv=2, D=16, L=(4, 30), steps=(3,))
    s = 3
    base, _ = oracle.attend(*_args(w))
    perm = np.random.default_rng(1).permutation(w.BW)  # slot b moves to perm[b]
    q = np.empty_like(w.q[0])
    q[:, perm] = w.q[0]
    uk, uv, par = w.unshared_k.copy(), w.unshared_v.copy(), w.parent_idx.copy()
    uk[:, :, s, perm] = w.unshared_k[:, :, s]
    uv[:, :, s, perm] = w.unshared_v[:, :, s]
    par[:, s, perm] = w.parent_idx[:, s]
    out, _ = oracle.attend(q, w.shared_k, w.shared_v, w.prompt_len, uk, uv, par, s)
    assert np.max(np.abs(out[:, perm] - base)) <= TOL


def test_invalid_arguments_raise():
    w = _wl(seed=35)
    q, sk, sv, pl, uk, uv, par, s = _args(w)
    bad = pl.copy()
    bad[0] = w.Lmax + 1
    with pytest.raises(ValueError):
        oracle.attend(q, sk, sv, bad, uk, uv, par, s)
    with pytest.raises(ValueError):
        oracle.attend(q, sk, sv, pl, uk, uv, par, w.S)
