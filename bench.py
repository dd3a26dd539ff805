#!/usr/bin/env python3
"""Benchmark of staged beam-search decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--G g]

One benchmark step is one pass of the whole path over one batch of the
workload: for the default large-batch workload (64 requests, 2048-token
prompts, 256 beams with skewed branching, 3 decode steps, 32 query / 8 KV
heads, head_dim 128, bf16) that is 3 calls of xattn_decode, levels 0, 1, 2.
Inputs are resident in HBM before timing starts; enough distinct copies of
them are rotated (>= 1 GB) that timed calls read HBM rather than the 256 MB
Infinity Cache.

Prints ONE JSON line.  `value` is beam-steps per second over the timed
region (wall clock between two device synchronisations).  `roofline` covers
the decode kernel: algorithmic bytes (unique KV rows + q + out + indices) or
FLOPs per launch divided by the kernel's mean launch duration, measured with
a pair of HIP events bound to the kernel dispatch (xattn_decode_timed), so
the duration is the kernel's own, as a kernel trace reports it.  The events
are bound to the calls of every n-th step of the timed region (--time-every,
default 4): their markers cost the GPU about 4 us per launch, which binding
them to every call would charge to the throughput.
`cpu_baseline` times the float64 CPU oracle on the host cores on a bounded
sample of the same workload.  After the timed region, `other_workloads`
measures the other workloads the same way with fewer steps (GR serving,
wide beam, and the prefix-homogeneity sweep at every group size), and side
legs time other kernels on the same device: `per_beam_comparison` (the per-beam
PagedAttention-style kernel on the same inputs), `beam_selection` (the
top-BW beam selection on the workload's BW x BW candidate pool),
`unshared_reorder` (the in-place Unshared-cache reorder at each level) and
`valid_path_mask` (masking the workload's beams' logits over a 2^20-item
vocabulary at each depth).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention beam-steps/sec + achieved HBM GB/s (unique KV bytes) vs peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FP32_VECTOR_PEAK_TFLOPS = 157.3
# everything that decides the device code: the HIP sources, the headers and
# the build flags
CODE_GLOBS = ("generative_recommendation_beam_xattn_amd/csrc/*", "include/*.h",
              "generative_recommendation_beam_xattn_amd/build.py")
# what the main line measures when no --config is given: the largest
# single-GPU workload (64 requests x 256 beams, 2048-token prompts)
DEFAULT_CONFIG = 3
SIDE_WORKLOADS = [(2, None), (4, None), (5, 1), (5, 8), (5, 32), (5, 256)]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--G", type=int, default=None, help="prefix group size for config 5")
    ap.add_argument("--rot", type=int, default=None, help="rotation copies (default: >= 1 GB)")
    ap.add_argument("--time-every", type=int, default=4,
                    help="bind timing events to the calls of every n-th timed step (the events "
                         "cost the GPU about 4 us per launch, so binding them to every call would "
                         "charge them to the throughput)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--per-beam-steps", type=int, default=10,
                    help="steps of the per-beam comparison kernel timed after the main run "
                         "(0 skips it)")
    ap.add_argument("--topk-steps", type=int, default=50,
                    help="launches of beam selection (xattn_beam_topk) timed after the main run "
                         "on the workload's BW x BW candidate pool (0 skips it)")
    ap.add_argument("--reorder-steps", type=int, default=20,
                    help="rounds of the in-place Unshared reorder timed after the main run, on "
                         "the rotation copies (0 skips it)")
    ap.add_argument("--mask-steps", type=int, default=20,
                    help="rounds of valid-path masking timed after the main run, per depth, on "
                         "the workload's beams over the full item vocabulary (0 skips it)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak leg (a 1 GiB device copy and the "
                         "matrix-core probe)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--side-steps", type=int, default=40,
                    help="timed steps of each other workload (0 skips them)")
    return ap.parse_args()


# ----------------------------------------------------------------- accounting

def distinct_ancestor_rows(parent_idx_r: np.ndarray, step: int) -> int:
    """Sum over levels 0..step of the number of distinct slots any beam reaches."""
    BW = parent_idx_r.shape[1]
    live = np.arange(BW)
    total = 0
    for t in range(step, -1, -1):
        live = np.unique(live)
        total += live.size
        if t >= 1:
            live = parent_idx_r[t][live]
    return total


def algorithmic_work(w, step_index: int) -> dict:
    """Compulsory bytes and FLOPs of one xattn_decode call."""
    s = w.steps[step_index]
    e = w.elem_bytes
    row_bytes = w.D * e
    shared_rows = int(np.sum(w.prompt_len)) * w.Hkv
    unshared_rows = sum(distinct_ancestor_rows(w.parent_idx[r], s) for r in range(w.R)) * w.Hkv
    kv_bytes = 2 * row_bytes * (shared_rows + unshared_rows)   # K and V
    q_bytes = w.R * w.BW * w.Hq * row_bytes
    idx_bytes = w.R * s * w.BW * 4 + w.R * 4
    G = w.Hq // w.Hkv
    flops = 4 * w.D * G * w.BW * w.Hkv * int(np.sum(w.prompt_len.astype(np.int64) + s + 1))
    return {"unique_kv_bytes": kv_bytes, "q_out_bytes": 2 * q_bytes, "index_bytes": idx_bytes,
            "bytes": kv_bytes + 2 * q_bytes + idx_bytes, "flops": flops}


def workload_config(w, n_rot: int) -> dict:
    c = {"workload": w.name, "requests": w.R, "beam_width": w.BW, "q_heads": w.Hq,
         "kv_heads": w.Hkv, "head_dim": w.D, "decode_steps": list(w.steps),
         "calls_per_step": len(w.steps), "rotation_copies": n_rot}
    lo, hi = int(w.prompt_len.min()), int(w.prompt_len.max())
    c["prompt_len"] = lo if lo == hi else "uniform [%d, %d] (drawn %d..%d)" % (
        {2: 512}.get(w.meta.get("config"), lo), {2: 1024}.get(w.meta.get("config"), hi), lo, hi)
    if w.meta.get("G"):
        c["prefix_group"] = w.meta["G"]
    return c


def code_digest() -> str:
    """Digest of every file that decides the device code (sources, headers,
    build flags), in path order."""
    import glob
    h = hashlib.sha256()
    for pattern in CODE_GLOBS:
        for path in sorted(glob.glob(os.path.join(ROOT, pattern))):
            if path.endswith((".hip", ".h", ".py")):
                h.update(os.path.relpath(path, ROOT).encode())
                with open(path, "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(w):
    """Counter-measured HBM bytes per launch (profiles/traffic_<workload>.json,
    FETCH_SIZE + WRITE_SIZE scaled by a copy of known size), or None unless
    they were taken on exactly the current device code."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("code_sha256_16") != code_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def data_label(w) -> str:
    c = w.meta.get("config")
    kind = {1: "tiny plumbing", 2: "GR serving", 3: "large batch", 4: "wide beam",
            5: "prefix-homogeneity sweep"}.get(c, w.name)
    return "synthetic (seeded N(0,1), %s workload shape: %s)" % (kind, w.name)


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline(w, target_s: float) -> dict:
    """Float64 oracle throughput on this host, over whole passes of the workload
    ((request, decode step) pairs in order, repeated) until ~target_s of CPU time."""
    import oracle
    t_total, beam_steps, n_pairs = 0.0, 0, 0
    order = [(r, i) for r in range(w.R) for i in range(len(w.steps))]
    while t_total < target_s:
        for r, i in order:
            sl = slice(r, r + 1)
            t0 = time.perf_counter()
            oracle.attend(w.q[i][sl], w.shared_k[sl], w.shared_v[sl], w.prompt_len[sl],
                          w.unshared_k[sl], w.unshared_v[sl], w.parent_idx[sl], w.steps[i])
            t_total += time.perf_counter() - t0
            beam_steps += w.BW
            n_pairs += 1
            if t_total >= target_s:
                break
    # beam selection on the workload's BW x BW pool, for the beam_selection leg
    from generative_recommendation_beam_xattn_amd import workloads as W
    BW = min(w.BW, 512)
    pool = W.beam_pool(100 + w.meta.get("config", 0), w.R, BW, BW)
    reps, t_sel = 0, 0.0
    while t_sel < 1.0 and reps < 50:
        t0 = time.perf_counter()
        oracle.beam_topk(pool.cum, pool.logp, pool.token)
        t_sel += time.perf_counter() - t0
        reps += 1
    return {"value": beam_steps / t_total, "unit": "beam-steps/s", "cores": oracle.omp_threads(),
            "beam_selection_us_per_launch": t_sel / reps * 1e6,
            "kind": "oracle",
            "sample": "%d (request, decode step) pairs of the %s workload (%d per full pass), %d "
                      "beams each, %.1f s of float64 oracle time" % (
                          n_pairs, w.name, len(order), w.BW, t_total)}


# ------------------------------------------------------- Unshared-cache reorder

def reorder_bytes(parent: np.ndarray, Hkv: int, row_bytes: int, levels: int) -> int:
    """Compulsory bytes of one in-place reorder of `levels` levels with
    parents `parent` [R][BW]: per request, every row whose parent is another
    slot is written, and every distinct slot such a row takes its history
    from is read, at each level, K and V, for every KV head."""
    par = np.asarray(parent)
    mv = par != np.arange(par.shape[1])[None, :]
    moved = int(mv.sum())
    sources = sum(int(np.unique(par[r][mv[r]]).size) for r in range(par.shape[0]))
    return 2 * Hkv * levels * row_bytes * (sources + moved)


def reorder_leg(w, copies, steps: int, stream) -> dict | None:
    """xattn_reorder_unshared as a caller would run it after each selection:
    at every decode level s >= 1 of the workload, levels 0..s-1 take the
    rows of parent_idx[:, s, :].  Timed per launch with events bound to the
    dispatch.  Each launch works on the next of a rotation of Unshared
    caches holding >= 1 GiB together (the decode run's copies, plus clones
    where those hold less), so that no launch finds its rows in the 256 MB
    last-level cache.  Algorithmic bytes, K and V: every row that moves
    written once, and every distinct row it takes its history from read once
    (rows that keep their place are neither read nor written)."""
    import torch
    from generative_recommendation_beam_xattn_amd import binding as B
    levels = [s for s in w.steps if s >= 1]
    if not levels or w.BW > 2048:
        return None
    per_set = 2 * copies[0]["uk"].numel() * copies[0]["uk"].element_size()
    n_sets = max(len(copies), math.ceil((1 << 30) / per_set))
    sets = [(c["uk"], c["uv"]) for c in copies]
    sets += [(copies[0]["uk"].clone(), copies[0]["uv"].clone())
             for _ in range(n_sets - len(copies))]
    par = copies[0]["par"]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in levels] for _ in range(steps + 1)]
    for row in ev:
        for a, b in row:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    n = 0
    for k in range(steps + 1):      # round 0 is a warmup
        for i, s in enumerate(levels):
            uk, uv = sets[n % n_sets]
            n += 1
            B.reorder_unshared(uk, uv, par[:, s, :], s, stream=stream, events=ev[k][i])
    torch.cuda.synchronize()
    del sets
    us = np.array([[a.elapsed_time(b) * 1e3 for a, b in ev[k]] for k in range(1, steps + 1)])
    row = w.D * w.elem_bytes
    by_level = []
    for i, s in enumerate(levels):
        byts = reorder_bytes(w.parent_idx[:, s, :], w.Hkv, row, s)
        t = float(us[:, i].mean())
        by_level.append({"level": s, "levels_moved": s, "kernel_us": t, "bytes": byts,
                         "GBps": byts / t / 1e3, "frac_of_hbm_peak": byts / t / 1e3 / HBM_PEAK_GBS})
    return {"by_level": by_level, "bound": "hbm", "steps": steps, "cache_sets": n_sets}


# ------------------------------------------------------------ valid-path masks

def valid_mask_leg(w, steps: int, dev, stream) -> dict | None:
    """xattn_valid_mask on R x BW beams of the workload over the full item
    vocabulary (2^20 items of 3 tokens over 8192 ids; dense masks at depths
    0 and 1, sparse at 2), at every depth, on logits rotated through enough
    buffers (>= 512 MB) to come from HBM.  Beams sit on prefixes of random
    items (one in ten random, mostly dead).  Algorithmic bytes per launch:
    4 B per slot that becomes -inf (valid slots are neither read nor
    written), and each distinct node's mask row (dense) or children (sparse)
    once."""
    import torch
    from generative_recommendation_beam_xattn_amd import binding as B
    from generative_recommendation_beam_xattn_amd import workloads as W
    c = W.VALID_ITEMS_FULL
    R, BW, V, L = w.R, w.BW, c["vocab"], c["levels"]
    items = W.valid_items(42, **c)
    vp = B.ValidPaths(items, V, 2, device=dev)
    rng = np.random.default_rng(5)
    row_bytes = R * BW * V * 4
    n_buf = max(2, min(16, -(-512 * 2**20 // row_bytes)))
    bufs = [torch.empty((R, BW, V), dtype=torch.float32, device=dev) for _ in range(n_buf)]
    for b in bufs:
        b.normal_()
    ident = torch.arange(BW, dtype=torch.int32, device=dev).repeat(R, 1).contiguous()
    pick = rng.integers(0, len(items), size=R * BW)
    rand = rng.random(R * BW) < 0.1
    paths = np.where(rand[:, None], rng.integers(0, V, size=(R * BW, L)), items[pick])
    node = vp.root(R, BW)
    out = []
    for depth in range(L):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps + 1)]
        for a, b in ev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        for k in range(steps + 1):       # round 0 is a warmup
            vp.mask(depth, node, bufs[k % n_buf], stream=stream, events=ev[k])
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev[1:]]) * 1e3)
        n_valid = int(torch.isfinite(bufs[0]).sum().item())
        nodes = np.unique(node.cpu().numpy())
        nodes = nodes[nodes >= 0]
        if depth < vp.layout.dense_levels:
            table_bytes = len(nodes) * vp.layout.words * 4
        else:
            table_bytes = 8 * len(nodes) + 4 * n_valid
        byts = 4 * (R * BW * V - n_valid) + table_bytes
        out.append({"depth": depth, "dense": depth < vp.layout.dense_levels, "kernel_us": us,
                    "valid_slots": n_valid, "bytes": byts, "GBps": byts / us / 1e3,
                    "frac_of_hbm_peak": byts / us / 1e3 / HBM_PEAK_GBS})
        tok = torch.from_numpy(paths[:, depth].astype(np.int32).reshape(R, BW)).to(dev)
        node = vp.advance(depth, node, ident, tok)
    torch.cuda.synchronize()
    return {"beams": {"R": R, "BW": BW}, "vocab": V, "items": c["n_items"],
            "by_depth": out, "bound": "hbm", "buffers": n_buf, "steps": steps}


# ------------------------------------------------------------ beam selection

def achievable_peaks_leg(dev, stream) -> dict:
    """What this chip delivers: the HBM read probe over 1 GiB
    (xattn_peak_read), a 1 GiB device-to-device copy (bytes read + written
    per second, for context) and the matrix-core probe (xattn_peak_mfma_bf16,
    independent bf16 MFMA chains on every SIMD), each the median of 5 timed
    runs after 2 untimed ones."""
    import torch
    from generative_recommendation_beam_xattn_amd import binding as B
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = []
    for k in range(7):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        if k >= 2:
            t_copy.append(a.elapsed_time(b) / 1e3)
    del dst
    t_read = []
    for k in range(7):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev:
            e.record(stream)
        B.peak_read(src, 8192, stream, ev)
        torch.cuda.synchronize()
        if k >= 2:
            t_read.append(ev[0].elapsed_time(ev[1]) / 1e3)
    del src
    blocks, iters = 1024, 4000      # 4 waves per SIMD on 256 CUs, about 1 ms
    t_mfma, flops = [], 0.0
    for k in range(7):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in ev:
            e.record(stream)
        flops, _ = B.peak_mfma_bf16(iters, blocks, stream, ev)
        torch.cuda.synchronize()
        if k >= 2:
            t_mfma.append(ev[0].elapsed_time(ev[1]) / 1e3)
    return {"hbm_read_GBps": float((1 << 30) / np.median(t_read) / 1e9),
            "hbm_copy_GBps": float(2 * (1 << 30) / np.median(t_copy) / 1e9),
            "mfma_bf16_TFLOPs": float(flops / np.median(t_mfma) / 1e12),
            "read": "xattn_peak_read: 1 GiB streamed once by 8192 workgroups, 16-byte "
                    "non-temporal loads",
            "copy": "1 GiB device-to-device copy, bytes read + written",
            "mfma": "xattn_peak_mfma_bf16: %d workgroups x 4 waves, %d rounds of 4 independent "
                    "v_mfma_f32_32x32x16_bf16 chains" % (blocks, iters)}


def beam_selection_leg(w, steps: int, dev) -> dict:
    """xattn_beam_topk on the workload's candidate pool: every beam proposes
    BW candidates (the BW x BW pools of the xGR summary), R requests per
    launch.  Per-launch kernel time from events bound to the dispatch; for
    scale, torch.topk over the flattened scores of the same pool (a
    different tie order, so only its time is reported)."""
    import torch
    from generative_recommendation_beam_xattn_amd import binding as B
    from generative_recommendation_beam_xattn_amd import workloads as W
    BW = min(w.BW, 512)
    pool = W.beam_pool(100 + w.meta.get("config", 0), w.R, BW, BW)
    cum = torch.from_numpy(pool.cum).to(dev)
    logp = torch.from_numpy(pool.logp).to(dev)
    tok = torch.from_numpy(pool.token).to(dev)
    out = B.beam_topk(cum, logp, tok)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for pair in ev:
        for e in pair:
            e.record()
    torch.cuda.synchronize()
    for pair in ev:
        B.beam_topk(cum, logp, tok, out=out, events=pair)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev]) * 1e3)
    flat = (cum[:, :, None] + logp).reshape(w.R, -1)
    for _ in range(3):
        torch.topk(flat, BW, dim=1)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        torch.topk(flat, BW, dim=1)
    b.record()
    torch.cuda.synchronize()
    n_cand = w.R * BW * BW
    return {"pool": {"R": w.R, "BW": BW, "V": BW}, "kernel_us_per_launch": us,
            "candidates_per_s": n_cand / (us * 1e-6), "selections_per_s": w.R * BW / (us * 1e-6),
            "bound": "latency (one workgroup per request)",
            "torch_topk_flat_us": float(a.elapsed_time(b) * 1e3 / steps), "steps": steps}


# ---------------------------------------------------------------------- main

def roofline_of(w, work, t_kernel: float) -> dict:
    """The binding roofline of one launch: algorithmic bytes (HBM) or FLOPs
    (matrix cores) per launch over the mean launch duration."""
    bytes_per_launch = float(np.mean([x["bytes"] for x in work]))
    flops_per_launch = float(np.mean([x["flops"] for x in work]))
    t_hbm = bytes_per_launch / (HBM_PEAK_GBS * 1e9)
    peak_c = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
    t_cmp = flops_per_launch / (peak_c * 1e12)
    if t_hbm >= t_cmp:
        roof = {"bound": "hbm", "achieved": bytes_per_launch / t_kernel / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu",
                "achieved": flops_per_launch / t_kernel / 1e12, "peak": peak_c,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["binding_frac"] = max(t_hbm, t_cmp) / t_kernel
    return roof


class Measured:
    """One workload on the device: rotation copies of every input, decode
    calls marshalled once, a timed region of whole steps (all decode levels
    of the workload) between two synchronisations, and each call's kernel
    duration from events bound to its dispatch on every n-th step."""

    def __init__(self, w, dev, rot=None):
        import torch
        from generative_recommendation_beam_xattn_amd import binding as B

        def to_dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        self.w = w
        self.n_calls = len(w.steps)
        self.work = [algorithmic_work(w, i) for i in range(self.n_calls)]
        copy_bytes = (w.q.nbytes * 2 + w.shared_k.nbytes * 2 + w.unshared_k.nbytes * 2 +
                      w.parent_idx.nbytes)
        self.n_rot = rot or max(1, min(32, math.ceil(1e9 / copy_bytes)))
        base = {"q": [to_dev(w.q[i]) for i in range(self.n_calls)], "sk": to_dev(w.shared_k),
                "sv": to_dev(w.shared_v), "pl": to_dev(w.prompt_len),
                "uk": to_dev(w.unshared_k), "uv": to_dev(w.unshared_v),
                "par": to_dev(w.parent_idx)}
        self.copies = [base] + [{k: ([t.clone() for t in v] if isinstance(v, list)
                                     else v.clone()) for k, v in base.items()}
                                for _ in range(self.n_rot - 1)]
        self.calls = [[B.PreparedDecode(c["q"][i], c["sk"], c["sv"], c["pl"], c["uk"], c["uv"],
                                        c["par"], w.steps[i]) for i in range(self.n_calls)]
                      for c in self.copies]

    def run(self, stream, steps: int, warmup: int, every: int):
        import torch
        n_calls, n_rot = self.n_calls, self.n_rot

        def run_step(k, events=None):
            for i, call in enumerate(self.calls[k % n_rot]):
                call(stream, None if events is None else (events[2 * i], events[2 * i + 1]))

        for k in range(warmup):
            run_step(k)
        timed_steps = [k for k in range(steps) if k % every == 0]
        ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_calls)]
              for k in timed_steps}
        for row in ev.values():   # torch creates the HIP event at its first record
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            run_step(warmup + k, ev.get(k))
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - t0
        self.steps = steps
        # per-launch durations (ms) of each decode call, by level
        self.per_call = np.array([[ev[k][2 * i].elapsed_time(ev[k][2 * i + 1])
                                   for i in range(n_calls)] for k in timed_steps])
        self.every = every
        return self

    def summary(self, with_traffic=True) -> dict:
        w = self.w
        mean_launch_s = self.per_call.mean(axis=0) / 1e3
        t_kernel = float(mean_launch_s.mean())
        roof = roofline_of(w, self.work, t_kernel)
        binding = roof.pop("binding_frac")
        roof["traffic"] = stored_traffic(w) if with_traffic else None
        ukv = float(np.mean([x["unique_kv_bytes"] for x in self.work]))
        rows = self.steps * self.n_calls * w.R * w.BW
        return {
            "value": rows / self.wall,
            "unit": "sequence-steps/s" if w.meta.get("config") == 5 else "beam-steps/s",
            "ms_per_step": self.wall / self.steps * 1e3,
            "steps": self.steps,
            "dtype": w.dtype,
            "data": data_label(w),
            "config": workload_config(w, self.n_rot),
            "roofline": roof,
            "unique_kv_GBps": ukv / t_kernel / 1e9,
            "unique_kv_frac_of_hbm_peak": ukv / t_kernel / 1e9 / HBM_PEAK_GBS,
            "binding_roofline_frac": binding,
            "kernel_us_per_launch": {"mean": t_kernel * 1e6,
                                     "by_level": [float(x * 1e6) for x in mean_launch_s],
                                     "p10": float(np.percentile(self.per_call, 10) * 1e3),
                                     "p50": float(np.percentile(self.per_call, 50) * 1e3),
                                     "p90": float(np.percentile(self.per_call, 90) * 1e3),
                                     "launches_timed": int(self.per_call.size),
                                     "every_nth_step": self.every},
            "algorithmic_per_launch": {
                "bytes": float(np.mean([x["bytes"] for x in self.work])),
                "unique_kv_bytes": ukv,
                "flops": float(np.mean([x["flops"] for x in self.work]))},
        }


def per_beam_leg(m, stream, steps: int) -> dict:
    """The per-beam (PagedAttention-style) comparison kernel on the same
    inputs, outside the timed region: its per-launch duration, as the staged
    one's."""
    import torch
    from generative_recommendation_beam_xattn_amd import binding as B
    w = m.w
    pb_calls = [[B.PreparedDecode(c["q"][i], c["sk"], c["sv"], c["pl"], c["uk"], c["uv"],
                                  c["par"], w.steps[i], per_beam=True)
                 for i in range(m.n_calls)] for c in m.copies]
    pb_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * m.n_calls)]
             for _ in range(steps + 1)]
    for row in pb_ev:
        for e in row:
            e.record(stream)
    for k in range(steps + 1):   # the first step is a warmup
        for i, call in enumerate(pb_calls[k % m.n_rot]):
            call(stream, (pb_ev[k][2 * i], pb_ev[k][2 * i + 1]))
    torch.cuda.synchronize()
    pb = np.array([[pb_ev[k][2 * i].elapsed_time(pb_ev[k][2 * i + 1]) for i in range(m.n_calls)]
                   for k in range(1, steps + 1)])
    pb_us = float(pb.mean() * 1e3)
    return {"kernel_us_per_launch": pb_us,
            "staged_speedup": pb_us / (float(m.per_call.mean()) * 1e3),
            "prompt_bytes_read_per_launch": float(
                2 * w.elem_bytes * w.D * w.Hkv * w.BW * int(np.sum(w.prompt_len))),
            "steps": steps}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: one GPU only; --gpus %d is not supported.  The path shards "
              "by request or KV head with no exchange, so N GPUs would each run this kernel on "
              "their share." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from generative_recommendation_beam_xattn_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    every = max(1, args.time_every)

    w = W.make(args.config, args.G)
    m = Measured(w, dev, args.rot).run(stream, args.steps, args.warmup, every)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per_beam = per_beam_leg(m, stream, args.per_beam_steps) if args.per_beam_steps > 0 else None
    peaks = None if args.no_peaks else achievable_peaks_leg(dev, stream)
    beam_sel = beam_selection_leg(w, args.topk_steps, dev) if args.topk_steps > 0 else None
    reorder = (reorder_leg(w, m.copies, args.reorder_steps, stream)
               if args.reorder_steps > 0 else None)
    masks = valid_mask_leg(w, args.mask_steps, dev, stream) if args.mask_steps > 0 else None

    head = m.summary()
    if peaks is not None:
        # the same achieved rate against what this chip delivers (published
        # peaks assume the top clock and an ideal memory system)
        roof = head["roofline"]
        ref = {"hbm": peaks["hbm_read_GBps"], "mfma": peaks["mfma_bf16_TFLOPs"]}.get(roof["bound"])
        peaks["roofline_frac_of_achievable"] = roof["achieved"] / ref if ref else None
    del m
    torch.cuda.empty_cache()

    # the other workloads, each measured the same way on fewer steps
    others = []
    if args.side_steps > 0:
        for cfg, G in SIDE_WORKLOADS:
            if (cfg, G) == (args.config, args.G):
                continue
            ws = W.make(cfg, G)
            ms = Measured(ws, dev).run(stream, args.side_steps, max(5, args.side_steps // 4), every)
            sm = ms.summary()
            if per_beam is not None and cfg != 5:
                sm["per_beam_comparison"] = per_beam_leg(ms, stream, 3)
            others.append(sm)
            del ms, ws
            torch.cuda.empty_cache()
            print("bench: %s done" % sm["config"]["workload"], file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": head["data"],
        "config": head["config"],
        "roofline": head["roofline"],
        "unique_kv_GBps": head["unique_kv_GBps"],
        "unique_kv_frac_of_hbm_peak": head["unique_kv_frac_of_hbm_peak"],
        "binding_roofline_frac": head["binding_roofline_frac"],
        "kernel_us_per_launch": head["kernel_us_per_launch"],
        "algorithmic_per_launch": head["algorithmic_per_launch"],
        "code_sha256_16": code_digest(),
        "cpu_baseline": None,
        "achievable_peaks": peaks,
        "per_beam_comparison": per_beam,
        "other_workloads": others,
        "beam_selection": beam_sel,
        "unshared_reorder": reorder,
        "valid_path_mask": masks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
