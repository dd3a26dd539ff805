"""The seeded tiny workload and the oracle's values on it are stable (no GPU)."""
import json
import os

import numpy as np

import oracle
from generative_recommendation_beam_xattn_amd import workloads as W
from tests.golden.make_golden import digests

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def test_tiny_workload_stream_is_stable():
    doc = json.load(open(GOLDEN))
    assert digests(W.make(1)) == doc["digests"]


def test_tiny_oracle_values_are_stable():
    doc = json.load(open(GOLDEN))
    w = W.make(1)
    for i, st in enumerate(doc["steps"]):
        out, lse = oracle.attend(w.q[i], w.shared_k, w.shared_v, w.prompt_len, w.unshared_k,
                                 w.unshared_v, w.parent_idx, st["step"])
        got = [out[0, b, h, d] for b, h, d in doc["positions_b_h_d"]]
        assert np.max(np.abs(np.array(got) - np.array(st["out"]))) <= 1e-12
        assert oracle.ancestors(w.parent_idx, st["step"])[0].tolist() == st["anc"]
