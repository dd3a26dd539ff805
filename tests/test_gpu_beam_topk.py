"""GPU parity of beam selection (xattn_beam_topk) against the oracle.

The outputs are integers decided by float32 scores computed the same way on
both sides (one float32 addition), so the bar is bit-exact: parent and token
ids equal, scores equal as floats.  Cases: small and full pool sizes (128 x
128 and 512 x 512), every input variant of the generator (ties, identical
rows, masked tails), dominant beams whose runs reach past the sampled
prefix, tie runs that continue to the end of a row, the beam-width and
vocabulary extremes, strided outputs written straight into a parent_idx
array, and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import generative_recommendation_beam_xattn_amd as X
from generative_recommendation_beam_xattn_amd import workloads as W
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_gpu(cum, logp, tok):
    out = X.beam_topk(to_dev(cum), to_dev(logp), to_dev(tok))
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in out)


def check(cum, logp, tok, name):
    R, BW, V = logp.shape
    say("[%s] beam_topk R=%d BW=%d V=%d" % (name, R, BW, V))
    s, p, t = run_gpu(cum, logp, tok)
    rs, rp, rt = oracle.beam_topk(cum, logp, tok)
    for r in range(R):
        bad = np.nonzero((p[r] != rp[r]) | (t[r] != rt[r]) | (s[r] != rs[r]))[0]
        assert bad.size == 0, "%s request %d: first mismatch at %d: gpu (%r, %d, %d) oracle " \
            "(%r, %d, %d)" % (name, r, bad[0], s[r, bad[0]], p[r, bad[0]], t[r, bad[0]],
                               rs[r, bad[0]], rp[r, bad[0]], rt[r, bad[0]])


SHAPES = [(1, 1, 1), (2, 1, 7), (3, 4, 1), (3, 7, 33), (2, 16, 64), (2, 64, 65), (2, 100, 200),
          (2, 128, 128), (1, 256, 300), (2, 511, 40), (1, 512, 1), (1, 512, 97)]
VARIANTS = [("normal", 0.0), ("ties", 0.0), ("identical", 0.0), ("normal", 0.9), ("ties", 0.5)]


@pytest.mark.parametrize("kind,masked", VARIANTS)
@pytest.mark.parametrize("R,BW,V", SHAPES)
def test_small_pools(R, BW, V, kind, masked):
    p = W.beam_pool(1000 + BW * 7 + V, R, BW, V, kind=kind, masked_frac=masked)
    check(p.cum, p.logp, p.token, "small-%s-%g" % (kind, masked))


@pytest.mark.parametrize("pool", sorted(W.BEAM_POOLS))
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_full_pools(pool, kind):
    c = W.BEAM_POOLS[pool]
    p = W.beam_pool(17, c["R"], c["BW"], c["V"], kind=kind)
    check(p.cum, p.logp, p.token, pool + "-" + kind)


@pytest.mark.parametrize("BW,V", [(128, 128), (512, 512), (64, 700), (300, 1000)])
def test_dominant_beams(BW, V):
    # a few beams far ahead: their selected runs reach past the sampled
    # prefix, and the candidates above the sample threshold must be gathered
    p = W.beam_pool(5 + BW, 2, BW, V)
    cum = p.cum.copy()
    cum[0, : max(1, BW // 40)] += 60.0
    cum[1, BW // 2] += 200.0
    check(cum, p.logp, p.token, "dominant")


@pytest.mark.parametrize("BW,V", [(64, 700), (512, 600), (16, 2000), (200, 100)])
def test_tie_runs_to_row_end(BW, V):
    # almost every candidate masked: the threshold is -inf and the tie runs
    # extend to the end of the rows, past everything sampled
    p = W.beam_pool(9 + V, 2, BW, V)
    logp = p.logp.copy()
    logp[:, :, 1:] = -np.inf
    logp[:, ::2, :] = -np.inf
    check(p.cum, logp, p.token, "masked-runs")


@pytest.mark.parametrize("BW,V", [(128, 128), (512, 512), (33, 777)])
def test_flat_rows_and_negative_tokens(BW, V):
    p = W.beam_pool(21, 2, BW, V)
    logp = (np.round(p.logp / 8) * 8).astype(np.float32)   # long equal runs
    cum = np.round(p.cum).astype(np.float32)
    tok = (p.token - 4096).astype(np.int32)                # signed ids order too
    check(cum, logp, tok, "flat")


def test_float32_rounding_tie():
    cum = np.array([[1e8, -1e9]], np.float32)
    logp = np.array([[[-1.0, -2.0], [-1.0, -2.0]]], np.float32)
    tok = np.array([[[5, 3], [1, 2]]], np.int32)
    s, p, t = run_gpu(cum, logp, tok)
    np.testing.assert_array_equal(s[0], [1e8, 1e8])
    np.testing.assert_array_equal(p[0], [0, 0])
    np.testing.assert_array_equal(t[0], [3, 5])


def test_writes_into_parent_history_rows():
    # out_stride = S * BW: the parents land in row t of a parent_idx array
    R, BW, V, S, t = 4, 128, 128, 5, 3
    p = W.beam_pool(31, R, BW, V)
    dev = torch.device("cuda")
    hist_parent = torch.full((R, S, BW), -7, dtype=torch.int32, device=dev)
    hist_token = torch.full((R, S, BW), -7, dtype=torch.int32, device=dev)
    hist_score = torch.full((R, S, BW), -7.0, dtype=torch.float32, device=dev)
    X.beam_topk(to_dev(p.cum), to_dev(p.logp), to_dev(p.token),
                out=(hist_score[:, t, :], hist_parent[:, t, :], hist_token[:, t, :]))
    torch.cuda.synchronize()
    rs, rp, rt = oracle.beam_topk(p.cum, p.logp, p.token)
    hp, ht, hs = hist_parent.cpu().numpy(), hist_token.cpu().numpy(), hist_score.cpu().numpy()
    np.testing.assert_array_equal(hp[:, t], rp)
    np.testing.assert_array_equal(ht[:, t], rt)
    np.testing.assert_array_equal(hs[:, t], rs)
    others = [i for i in range(S) if i != t]
    assert (hp[:, others] == -7).all() and (ht[:, others] == -7).all()
    assert (hs[:, others] == -7.0).all()


def test_deterministic():
    c = W.BEAM_POOLS["wide_beam"]
    p = W.beam_pool(3, c["R"], c["BW"], c["V"], kind="ties")
    a = run_gpu(p.cum, p.logp, p.token)
    b = run_gpu(p.cum, p.logp, p.token)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


def test_timed_entry_matches():
    c = W.BEAM_POOLS["gr_serving"]
    p = W.beam_pool(4, c["R"], c["BW"], c["V"])
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    out = X.beam_topk(to_dev(p.cum), to_dev(p.logp), to_dev(p.token), events=ev)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    rs, rp, rt = oracle.beam_topk(p.cum, p.logp, p.token)
    np.testing.assert_array_equal(out[1].cpu().numpy(), rp)
    np.testing.assert_array_equal(out[2].cpu().numpy(), rt)
    np.testing.assert_array_equal(out[0].cpu().numpy(), rs)
