"""Write tests/golden/tiny_oracle.json (run: python tests/golden/make_golden.py).

The reference pages print no worked example, so this fixture is not an
independent pin: it records (a) SHA-256 digests of the seeded tiny workload
(1 request, prompt 128, 4 beams, 3 decode steps, 4/4 heads, head_dim 64,
fp32) so a change in the input stream is noticed, and (b) oracle outputs at
a fixed sample of positions, so a later change to the oracle's arithmetic is
noticed too.  Values come only from oracle/ on inputs from the workload
generator.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from generative_recommendation_beam_xattn_amd import workloads as W  # noqa: E402


def digests(w):
    return {k: hashlib.sha256(np.ascontiguousarray(getattr(w, k)).tobytes()).hexdigest()
            for k in ("prompt_len", "q", "shared_k", "shared_v", "unshared_k", "unshared_v",
                      "parent_idx")}


def sample_positions(w, n=24, seed=99):
    rng = np.random.default_rng(seed)
    return [[int(rng.integers(0, w.BW)), int(rng.integers(0, w.Hq)), int(rng.integers(0, w.D))]
            for _ in range(n)]


def main():
    w = W.make(1)
    pos = sample_positions(w)
    steps = []
    for i, s in enumerate(w.steps):
        out, lse = oracle.attend(w.q[i], w.shared_k, w.shared_v, w.prompt_len, w.unshared_k,
                                 w.unshared_v, w.parent_idx, s)
        anc = oracle.ancestors(w.parent_idx, s)
        steps.append({"step": s,
                      "out": [float(out[0, b, h, d]) for b, h, d in pos],
                      "lse": [float(lse[0, b, h]) for b, h, _ in pos],
                      "anc": anc[0].tolist()})
    doc = {"workload": "tiny (seed 1)", "digests": digests(w), "positions_b_h_d": pos,
           "steps": steps,
           "note": "oracle regression values; independent pins are in tests/test_oracle_pins.py"}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
