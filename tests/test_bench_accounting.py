"""The benchmark's algorithmic work per call, against independent counts.

Unique-KV bytes count every prompt row once per (request, KV head) and every
distinct generated-token (level, slot) row that some beam's history reaches
once, for K and V.  Here the distinct rows come from beam histories
simulated forward by copying (tests/brute.py), not from the backward walk
the benchmark uses; FLOPs are summed query row by query row.
"""
import numpy as np
import pytest

import bench
from generative_recommendation_beam_xattn_amd import workloads as W
from tests.brute import histories


def distinct_rows_forward(parent_idx_r, step):
    """parent_idx_r: one request's [S][BW] parent rows."""
    hist = histories(parent_idx_r[None], step)[0]
    return len({pair for h in hist for pair in h})


@pytest.mark.parametrize("seed,BW,step,kind", [(0, 4, 0, "uniform"), (1, 6, 3, "uniform"),
                                               (2, 16, 5, "uniform"), (3, 32, 2, "skewed"),
                                               (4, 8, 7, "identity")])
def test_distinct_ancestor_rows_match_forward_histories(seed, BW, step, kind):
    w = W.custom(seed=seed, R=3, L=5, BW=BW, steps=[step], Hq=2, Hkv=1, D=64, dtype="f32",
                 parents=kind)
    for r in range(w.R):
        assert bench.distinct_ancestor_rows(w.parent_idx[r], step) == \
            distinct_rows_forward(w.parent_idx[r], step)


def test_identity_parents_reach_every_row_and_constant_rows_one():
    BW, S = 5, 4
    ident = np.tile(np.arange(BW, dtype=np.int32), (S, 1))
    assert bench.distinct_ancestor_rows(ident, S - 1) == BW * S
    const = np.zeros((S, BW), np.int32)   # every beam descends from slot 0
    assert bench.distinct_ancestor_rows(const, S - 1) == BW + (S - 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_algorithmic_work_row_by_row(dtype):
    w = W.custom(seed=7, R=3, L=[10, 0, 33], BW=5, steps=[0, 2], Hq=6, Hkv=2, D=64,
                 dtype=dtype, S=3)
    e = 2 if dtype == "bf16" else 4
    for i, s in enumerate(w.steps):
        work = bench.algorithmic_work(w, i)
        flops = 0
        kv_rows = 0
        for r in range(w.R):
            L = int(w.prompt_len[r])
            for b in range(w.BW):
                for h in range(w.Hq):
                    flops += 4 * w.D * (L + s + 1)   # q.k and p.v per key
            kv_rows += w.Hkv * (L + distinct_rows_forward(w.parent_idx[r], s))
        assert work["flops"] == flops
        assert work["unique_kv_bytes"] == 2 * kv_rows * w.D * e
        q_bytes = w.R * w.BW * w.Hq * w.D * e
        assert work["bytes"] == work["unique_kv_bytes"] + 2 * q_bytes + work["index_bytes"]


def test_stored_traffic_only_for_the_code_it_was_measured_on(tmp_path, monkeypatch):
    """roofline.traffic comes from profiles/traffic_<workload>.json only while
    the digest of the device code (HIP sources, headers, build flags) matches
    the one recorded with the counters."""
    w = W.custom(name="traffic_probe", seed=0, R=1, L=4, BW=2, steps=[0], Hq=2, Hkv=1, D=64,
                 dtype="f32")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "traffic_traffic_probe.json"
    assert bench.stored_traffic(w) is None                  # no record
    digest = bench.code_digest()                            # of the (empty) tmp tree
    path.write_text('{"code_sha256_16": "%s", "hbm_bytes_per_launch": 123.0}' % digest)
    assert bench.stored_traffic(w) == 123.0
    path.write_text('{"code_sha256_16": "0000000000000000", "hbm_bytes_per_launch": 123.0}')
    assert bench.stored_traffic(w) is None                  # taken on other code


def test_code_digest_covers_sources_headers_and_build_flags(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "generative_recommendation_beam_xattn_amd" / "csrc"
    src.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    files = [src / "api.hip", src / "xattn_internal.h", tmp_path / "include" / "xattn.h",
             tmp_path / "generative_recommendation_beam_xattn_amd" / "build.py"]
    for f in files:
        f.write_text("a")
    base = bench.code_digest()
    for f in files:
        f.write_text("b")
        assert bench.code_digest() != base, f.name
        f.write_text("a")
    assert bench.code_digest() == base


def test_data_label_names_each_workload():
    labels = {bench.data_label(W.make(c, G, R=1)) for c, G in [(2, None), (3, None), (4, None)]}
    assert len(labels) == 3
    assert all(lbl.startswith("synthetic") for lbl in labels)


@pytest.mark.parametrize("seed", range(4))
def test_reorder_bytes_count_moved_rows_and_distinct_sources(seed):
    # brute force: walk every slot, collect the rows written and the rows read
    rng = np.random.default_rng(seed)
    R, BW, Hkv, row, levels = 3, 9, 2, 256, 2
    par = rng.integers(0, BW, size=(R, BW)).astype(np.int32)
    par[0] = np.arange(BW)                     # a request whose beams all stay
    par[1, :4] = np.arange(4)                  # some stay, the rest move
    written = read = 0
    for r in range(R):
        srcs = set()
        for b in range(BW):
            if par[r, b] != b:
                written += 1
                srcs.add(int(par[r, b]))
        read += len(srcs)
    want = 2 * Hkv * levels * row * (written + read)
    assert bench.reorder_bytes(par, Hkv, row, levels) == want
    assert bench.reorder_bytes(np.tile(np.arange(BW), (R, 1)), Hkv, row, levels) == 0
    # every beam from one parent: BW - 1 rows written, one row read
    one = np.zeros((1, BW), np.int32)
    assert bench.reorder_bytes(one, 1, row, 1) == 2 * row * (BW - 1 + 1)
