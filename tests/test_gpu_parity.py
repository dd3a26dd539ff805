"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars: max abs error <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs
(fp32 accumulation, bf16 output); ancestor slots bit-exact.  Small shapes
span several 64-key tiles, ragged tails of keys and query rows, every tiling
the launcher picks, deep parent chains and the degenerate cases.  The full
workload sizes are checked on every output row, in the launch configuration
the benchmark times, with the ancestor slots the decode path itself walked;
variants of them make the Unshared stage carry the result (empty prompts,
and generated-token values scaled up), so that a wrong or missing ancestor
row cannot hide under the 2e-2 bar.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import generative_recommendation_beam_xattn_amd as X
from generative_recommendation_beam_xattn_amd import binding as B
from generative_recommendation_beam_xattn_amd import workloads as W
from tests.gpu_util import TOL, DeviceWorkload, host_args, sample_rows, to_dev, to_f64, workload

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def check_full(w, name):
    dw = DeviceWorkload(w)
    for i, s in enumerate(w.steps):
        say("[%s] decode step %d (R=%d BW=%d Hq=%d Hkv=%d D=%d S=%d %s)" % (
            name, s, w.R, w.BW, w.Hq, w.Hkv, w.D, w.S, w.dtype))
        out = X.decode(*dw.args(i))
        torch.cuda.synchronize()
        ref, _ = oracle.attend(*host_args(w, i))
        err = np.max(np.abs(to_f64(out) - ref))
        assert err <= TOL[w.dtype], "%s step %d: max abs err %g" % (name, s, err)


SMALL = {
    # name: workload kwargs
    "ragged_rows_1wave": dict(R=3, BW=5, Hq=8, Hkv=2, D=128, L=[0, 77, 200], steps=[0, 1, 2]),
    "two_rowblocks_4x1": dict(R=2, BW=40, Hq=8, Hkv=2, D=128, L=[129, 511], steps=[0, 2], S=3),
    "d64_2waves": dict(R=2, BW=17, Hq=6, Hkv=3, D=64, L=[64, 191], steps=[1]),
    "g1_4x1": dict(R=2, BW=70, Hq=2, Hkv=2, D=128, L=[300, 1], steps=[2]),
    "qb2_tiling": dict(R=64, BW=64, Hq=32, Hkv=8, D=128, L=(30, 150), steps=[1], S=2),
    "deep_chain_workspace": dict(R=2, BW=6, Hq=4, Hkv=2, D=128, L=[50, 0], steps=[39], S=40),
    "deep_chain_wide": dict(R=1, BW=300, Hq=4, Hkv=4, D=64, L=[65], steps=[20], S=24),
    # deep chains whose few workgroups split their prompt tiles: 4 splits
    # (the short request leaves split 0 without a tile and masks a ragged
    # tail), and 2 splits at head_dim 64
    "deep_key_splits_ragged": dict(R=2, BW=32, Hq=8, Hkv=2, D=128, L=[1000, 130], steps=[20],
                                   S=21),
    "deep_key_splits_d64": dict(R=1, BW=16, Hq=8, Hkv=1, D=64, L=[700], steps=[17], S=18),
    # chains long enough for the segmented ancestor walk: 3 segments of 64
    # levels, and 4 segments of 27 levels with more beams than threads
    "deep_segmented_walk": dict(R=2, BW=40, Hq=4, Hkv=2, D=128, L=[100, 20], steps=[150],
                                S=151),
    "deep_segmented_wide": dict(R=1, BW=300, Hq=2, Hkv=2, D=64, L=[40], steps=[100], S=101),
    # the ancestor walk under tile 0's latency (prompts of more than three
    # tiles, parent rows staged): 64-row workgroups, and head_dim 64
    "early_walk_rg2": dict(R=2, BW=12, Hq=8, Hkv=2, D=128, L=[700, 257], steps=[1, 2], S=3),
    "early_walk_d64": dict(R=2, BW=24, Hq=8, Hkv=2, D=64, L=[450, 300], steps=[2], S=3),
    "single_beam_empty_prompt": dict(R=2, BW=1, Hq=4, Hkv=1, D=128, L=[0, 0], steps=[0]),
    "no_shared_rows": dict(R=2, BW=3, Hq=4, Hkv=2, D=64, L=[0, 0], steps=[1], Lmax=0),
    # either side of the row count below which bf16 calls go to the per-beam
    # kernel (8 query rows per request and KV head)
    "rows8_per_beam_path": dict(R=3, BW=2, Hq=8, Hkv=2, D=128, L=[70, 0, 333], steps=[0, 2], S=3),
    "rows9_staged_path": dict(R=3, BW=3, Hq=6, Hkv=2, D=128, L=[70, 0, 333], steps=[0, 2], S=3),
    # one head per KV head, 136 beams, 16 levels with the parent rows staged:
    # 128 beams per workgroup fill the 160 KiB of LDS exactly
    "lds_budget_g1_bw136": dict(R=2, BW=136, Hq=2, Hkv=2, D=128, L=[300, 700], steps=[15], S=16),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(name, dtype):
    kw = dict(SMALL[name])
    w = W.custom(name=name, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, **kw)
    check_full(w, name + "/" + dtype)


# Shapes that take the paired variant (>= 512 workgroups of 128 query
# rows): prompt lengths through every 32-key tile boundary (0, 1, one
# tile, one key past it, two and three tiles, ...), D = 128 and 64, one head
# per KV head with the LDS full, a deep chain, and G = 3 (row blocks that
# split a beam)
_EDGES = [0, 1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 200, 257, 300, 511]
PAIRED = {
    "paired_ragged": dict(R=64, BW=40, Hq=16, Hkv=8, D=128, L=_EDGES * 4, steps=[0, 2], S=3),
    "paired_d64": dict(R=64, BW=40, Hq=16, Hkv=8, D=64, L=_EDGES * 4, steps=[1], S=2),
    "paired_g1_full_lds": dict(R=32, BW=136, Hq=8, Hkv=8, D=128, L=(40, 130), steps=[15],
                               S=16),
    "paired_g3": dict(R=64, BW=50, Hq=24, Hkv=8, D=128, L=(60, 200), steps=[2], S=3),
    "paired_deep_chain": dict(R=64, BW=40, Hq=16, Hkv=8, D=128, L=(0, 150), steps=[20], S=21),
}


@pytest.mark.parametrize("name", sorted(PAIRED))
def test_paired_variant_shapes(name):
    w = W.custom(name=name, seed=zlib.crc32(name.encode()) % 1000, dtype="bf16", **PAIRED[name])
    shape = B.Shape(w.R, w.BW, w.Hq, w.Hkv, w.D, w.Lmax, w.S, B.XATTN_BF16, 0.0)
    for s in w.steps:
        assert X.plan(shape, s).kernel == B.KERNEL_STAGED_BF16_PAIRED
    check_full(w, name)


def test_tiny_workload_all_steps():
    w = W.make(1)
    check_full(w, "tiny")


def check_every_row(w, i, name, dw=None):
    """Every output row of step index i, and the ancestor slots of the same
    call, against the oracle; the slots' entry gives out bit for bit."""
    dw = dw or DeviceWorkload(w)
    s = w.steps[i]
    say("[%s] decode step %d, every row (R=%d BW=%d Hq=%d Hkv=%d D=%d S=%d)" % (
        name, s, w.R, w.BW, w.Hq, w.Hkv, w.D, w.S))
    out = X.decode(*dw.args(i))
    out2, anc = X.decode_with_ancestors(*dw.args(i))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    want = oracle.ancestors(w.parent_idx, s).transpose(0, 2, 1)
    assert np.array_equal(anc.cpu().numpy(), want), "%s step %d: ancestor slots" % (name, s)
    ref, _ = oracle.attend(*host_args(w, i))
    err = np.max(np.abs(to_f64(out) - ref))
    say("[%s] step %d: max abs err %.3g" % (name, s, err))
    assert err <= TOL[w.dtype], "%s step %d: max abs err %g" % (name, s, err)
    assert torch.isfinite(out.float()).all()


# the serving workload at every step; the large-batch (skewed parents) and
# wide-beam workloads at their last step
FULL = [(2, 0), (2, 1), (2, 2), (3, 2), (4, 3)]


@pytest.mark.parametrize("config,i", FULL)
def test_full_size_every_row(config, i):
    check_every_row(workload(config), i, "config %d" % config)


@pytest.mark.parametrize("G", W.PREFIX_GROUPS)
def test_prefix_sweep_every_row(G):
    check_every_row(workload(5, G), 0, "prefix sweep G=%d" % G)


@pytest.mark.parametrize("config", [2, 3, 4])
def test_unshared_stage_carries_the_result_every_row(config):
    """Full-size shapes where the Unshared stage carries the result.  A
    quarter of the requests have no prompt: their out is the Unshared stage
    alone.  The others keep their prompts, with generated-token keys scaled
    by 8 so that a beam's own tokens take most of the softmax weight.
    Generated-token values are halved, which keeps |out| below ~2.4 (bf16
    rounding of out stays near 0.008).  Changing one level's parents moves
    every empty-prompt row and 50-80 % of the others by >= 0.08 (measured on
    the oracle), four times the bar: a wrong, missing or misplaced ancestor
    row cannot hide under it."""
    base = workload(config)
    w = W.Workload(**{k: getattr(base, k) for k in base.__dataclass_fields__})
    w.prompt_len = base.prompt_len.copy()
    w.prompt_len[::4] = 0
    has_prompt = (w.prompt_len > 0)[:, None, None, None, None]
    k = W.bf16_bits_to_f32(base.unshared_k)
    w.unshared_k = W.to_bf16_bits(np.where(has_prompt, k * np.float32(8), k))
    w.unshared_v = W.to_bf16_bits(W.bf16_bits_to_f32(base.unshared_v) * np.float32(0.5))
    check_every_row(w, len(w.steps) - 1, "config %d, Unshared-dominant" % config)


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_ancestors_from_the_decode_path(config):
    """The slots each step's own chain walk used (inside the attention
    kernel for these short chains), against the oracle's, every step."""
    w = W.make(config, R=min(W.CONFIGS[config]["R"], 8)) if config != 1 else W.make(1)
    dw = DeviceWorkload(w)
    for i, s in enumerate(w.steps):
        say("[config %d] decode_with_ancestors step %d" % (config, s))
        _, anc = X.decode_with_ancestors(*dw.args(i))
        torch.cuda.synchronize()
        assert np.array_equal(anc.cpu().numpy(),
                              oracle.ancestors(w.parent_idx, s).transpose(0, 2, 1))


@pytest.mark.parametrize("BW,G,S,step", [(40, 4, 40, 39), (300, 1, 101, 100), (6, 2, 40, 39),
                                         (2, 4, 30, 29), (3, 4, 20, 17)])
def test_deep_chain_ancestors_from_the_decode_path(BW, G, S, step):
    """Deep chains: the chunked walk (one segment) and the segmented walk
    (300 beams: segments of 27 levels), on the staged, per-beam (2 beams x 4
    heads) and f32 kernels, as xattn_decode runs them."""
    for dtype in ("bf16", "f32"):
        w = W.custom(name="deep", seed=BW + S, R=2, BW=BW, Hq=2 * G, Hkv=2, D=64, L=[70, 5],
                     steps=[step], S=S, dtype=dtype)
        dw = DeviceWorkload(w)
        say("[deep ancestors BW=%d G=%d step=%d %s]" % (BW, G, step, dtype))
        out, anc = X.decode_with_ancestors(*dw.args(0))
        torch.cuda.synchronize()
        assert np.array_equal(anc.cpu().numpy(),
                              oracle.ancestors(w.parent_idx, step).transpose(0, 2, 1))
        ref, _ = oracle.attend(*host_args(w, 0))
        assert np.max(np.abs(to_f64(out) - ref)) <= TOL[dtype]


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_ancestors_exact(config):
    """xattn_resolve_ancestors, the chunked walk kernel on its own."""
    w = W.make(config, R=min(W.CONFIGS[config]["R"], 8)) if config != 1 else W.make(1)
    par = to_dev(w.parent_idx)
    for s in w.steps:
        say("[config %d] resolve_ancestors step %d" % (config, s))
        anc = X.resolve_ancestors(par, s).cpu().numpy()
        assert np.array_equal(anc, oracle.ancestors(w.parent_idx, s))


@pytest.mark.parametrize("BW,S,step", [(1, 512, 511), (256, 512, 511), (7, 33, 32), (9000, 3, 2),
                                       (300, 64, 0)])
def test_ancestors_exact_random_chains(BW, S, step):
    rng = np.random.default_rng(BW + S)
    p = rng.integers(0, BW, size=(2, S, BW), dtype=np.int32)
    say("[ancestors] BW=%d S=%d step=%d" % (BW, S, step))
    anc = X.resolve_ancestors(to_dev(p), step).cpu().numpy()
    assert np.array_equal(anc, oracle.ancestors(p, step))


DEBUG = {
    "tiny": None,
    "bf16_ragged": dict(R=3, BW=5, Hq=8, Hkv=2, D=128, L=[0, 77, 200], steps=[2]),
    "bf16_rowblocks": dict(R=2, BW=40, Hq=8, Hkv=2, D=64, L=[129, 64], steps=[1]),
    "bf16_deep": dict(R=2, BW=6, Hq=4, Hkv=2, D=128, L=[50, 0], steps=[39], S=40),
    # the serving shape's tiling: prompts of more than three tiles (ancestor
    # walk under tile 0, token chunks copied inside the tile loop) and an
    # empty prompt, 128 beams, 4 query heads per KV head
    "bf16_serving_tiling": dict(R=3, BW=128, Hq=16, Hkv=4, D=128, L=[700, 0, 257], steps=[2]),
    "bf16_segmented_deep": dict(R=1, BW=40, Hq=4, Hkv=2, D=128, L=[100], steps=[150], S=151),
    # the paired variant (512 workgroups of 128 rows), short and deep chains
    "bf16_paired": dict(R=64, BW=40, Hq=16, Hkv=8, D=128, L=_EDGES * 4, steps=[2]),
    "bf16_paired_deep": dict(R=64, BW=40, Hq=16, Hkv=8, D=128, L=(0, 150), steps=[20], S=21),
    "f32_ragged": dict(R=2, BW=5, Hq=8, Hkv=2, D=128, L=[0, 130], steps=[2], dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(DEBUG))
def test_debug_stage_taps(name):
    w = W.make(1) if DEBUG[name] is None else W.custom(name=name, seed=7, **DEBUG[name])
    dw = DeviceWorkload(w)
    i = len(w.steps) - 1
    say("[debug %s] decode_debug step %d" % (name, w.steps[i]))
    out, lse, ml, o = X.decode_debug(*dw.args(i))
    out_fast = X.decode(*dw.args(i))
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    ref, ref_lse = oracle.attend(*host_args(w, i))
    part = oracle.stage_partials(*host_args(w, i))
    assert np.max(np.abs(to_f64(out) - ref)) <= tol
    assert np.max(np.abs(to_f64(out_fast) - ref)) <= tol
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= tol
    ml = ml.cpu().numpy().astype(np.float64)
    o = o.cpu().numpy().astype(np.float64)
    for s_idx, key in ((0, "shared"), (1, "unshared")):
        rml, ro = part[key + "_ml"], part[key + "_o"]
        empty = rml[..., 1] == 0
        assert np.array_equal(ml[s_idx][..., 1] == 0, empty)
        assert np.all(np.isneginf(ml[s_idx][..., 0][empty]))
        ne = ~empty
        assert np.max(np.abs(ml[s_idx][..., 0][ne] - rml[..., 0][ne]), initial=0) <= tol
        # l is a sum of exp terms, compare relatively
        rel = np.abs(ml[s_idx][..., 1][ne] - rml[..., 1][ne]) / rml[..., 1][ne]
        assert np.max(rel, initial=0) <= tol
        assert np.max(np.abs(o[s_idx] - ro)) <= tol


def test_never_reads_past_prompt_step_or_row_zero():
    w = W.custom(name="poison", seed=3, R=3, BW=6, Hq=8, Hkv=2, D=128, L=[5, 70, 0], steps=[1],
                 S=4, Lmax=96)
    ref, _ = oracle.attend(*host_args(w, 0))
    nan = np.uint16(0x7FC0)
    for a in (w.shared_k, w.shared_v):
        for r, L in enumerate(w.prompt_len):
            a[r, :, L:] = nan
    for a in (w.unshared_k, w.unshared_v):
        a[:, :, 2:] = nan
    w.parent_idx[:, 0] = 3      # row 0 is never followed
    dw = DeviceWorkload(w)
    say("[poison] decode step 1")
    out = X.decode(*dw.args(0))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert np.max(np.abs(to_f64(out) - ref)) <= TOL["bf16"]


def test_bitwise_deterministic_and_out_buffer_reuse():
    w = W.make(2, R=4)
    dw = DeviceWorkload(w)
    say("[determinism] config 2 (4 requests)")
    a = X.decode(*dw.args(1))
    out = torch.full_like(a, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        X.decode(*dw.args(1), out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("case", ["bf16_gr_serving", "f32_small", "bf16_deep_chain"])
def test_timed_entry_matches_decode(case):
    if case == "bf16_gr_serving":
        w, i = W.make(2, R=4), 2
    elif case == "f32_small":
        w, i = W.custom(name="t32", seed=7, R=2, BW=5, Hq=8, Hkv=2, D=64, L=[70, 130],
                        steps=[1], S=2, dtype="f32"), 0
    else:
        w, i = W.custom(name="tdeep", seed=8, R=2, BW=6, Hq=4, Hkv=2, D=128, L=[50, 90],
                        steps=[30], S=31), 0
    dw = DeviceWorkload(w)
    say("[timed %s] step %d" % (case, w.steps[i]))
    ref = X.decode(*dw.args(i))
    call = X.PreparedDecode(*dw.args(i)[:8])
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in evs:
        e.record(stream)
    out = call(stream, events=evs)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref,
                       out.view(torch.int16) if out.dtype == torch.bfloat16 else out)
    t = evs[0].elapsed_time(evs[1])
    assert 0.0 < t < 1000.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_per_beam_small_shapes(name, dtype):
    w = W.custom(name=name, seed=zlib.crc32(name.encode()) % 1000 + 101, dtype=dtype,
                 **SMALL[name])
    dw = DeviceWorkload(w)
    for i, s in enumerate(w.steps):
        say("[per-beam %s/%s] step %d" % (name, dtype, s))
        out = X.decode_per_beam(*dw.args(i))
        torch.cuda.synchronize()
        ref, _ = oracle.attend(*host_args(w, i))
        err = np.max(np.abs(to_f64(out) - ref))
        assert err <= TOL[w.dtype], "%s step %d: max abs err %g" % (name, s, err)


def test_per_beam_gr_serving_sampled_and_close_to_staged():
    w = workload(2)
    dw = DeviceWorkload(w)
    for i, s in enumerate(w.steps):
        say("[per-beam gr_serving] step %d" % s)
        out = X.decode_per_beam(*dw.args(i))
        staged = X.decode(*dw.args(i))
        torch.cuda.synchronize()
        rows = sample_rows(w, 64, seed=40 + i)
        ref, _ = oracle.attend(*host_args(w, i), rows=rows)
        got = to_f64(out)[rows[:, 0], rows[:, 1], rows[:, 2]]
        assert np.max(np.abs(got - ref)) <= TOL["bf16"]
        # both are within the bar of the exact result, so within twice it of each other
        assert np.max(np.abs(to_f64(out) - to_f64(staged))) <= 2 * TOL["bf16"]


def test_invalid_arguments_raise_before_launch():
    w = W.custom(name="inv", seed=1, R=1, BW=2, Hq=2, Hkv=1, D=128, L=[8], steps=[0], S=2)
    dw = DeviceWorkload(w)
    q, sk, sv, pl, uk, uv, par, _ = dw.args(0)
    with pytest.raises(X.XattnError) as e:
        X.decode(q, sk, sv, pl, uk, uv, par, 2)
    assert e.value.status == 1
    with pytest.raises(X.XattnError) as e:
        X.decode(q[..., :96].contiguous(), sk[..., :96].contiguous(), sv[..., :96].contiguous(),
                 pl, uk[..., :96].contiguous(), uv[..., :96].contiguous(), par, 0)
    assert e.value.status == 2
