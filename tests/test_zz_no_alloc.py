"""xattn_decode_noalloc (no workspace argument, nothing allocated) against
xattn_decode with a workspace, through the C ABI: the same kernels, so the
outputs are equal bit for bit.  Two calls in a row on the same scratch, the
second with a smaller input; a step whose workspace would not fit the
scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import generative_recommendation_beam_xattn_amd as X
from generative_recommendation_beam_xattn_amd import binding as B
from generative_recommendation_beam_xattn_amd import workloads as W
from tests.gpu_util import TOL, DeviceWorkload, host_args, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def check_against_decode(w, label):
    dw = DeviceWorkload(w)
    args = dw.args(0)
    shape = B.make_shape(args[0], args[1], args[4])
    need = B.workspace_size(shape, w.steps[0])
    say("[noalloc %s] step %d, workspace %d bytes" % (label, w.steps[0], need))
    assert need <= B.NOALLOC_SCRATCH_BYTES
    want = X.decode(*args)
    out = torch.full_like(want, float("nan"))
    X.decode_noalloc(*args, out=out)
    torch.cuda.synchronize()
    assert torch.equal(want.view(torch.int16), out.view(torch.int16)), label
    ref, _ = oracle.attend(*host_args(w, 0))
    assert np.max(np.abs(to_f64(out) - ref)) <= TOL[w.dtype]
    return need


def test_noalloc_equals_decode_two_calls_second_smaller():
    # deep chains (the scratch holds ancestor slots, the Unshared partials
    # and, for the first, the partials of 4 key splits), then a smaller one
    big = W.custom(name="na_big", seed=11, R=2, BW=32, Hq=8, Hkv=2, D=128, L=[1000, 130],
                   steps=[20], S=21)
    small = W.custom(name="na_small", seed=12, R=1, BW=6, Hq=4, Hkv=2, D=64, L=[50],
                     steps=[39], S=40)
    n1 = check_against_decode(big, "big")
    n2 = check_against_decode(small, "small")
    assert 0 < n2 < n1


def test_noalloc_short_chain_and_sweep_shape():
    # no workspace needed: the scratch is not used at all
    w = W.make(2, R=2)
    w.steps = [2]
    w.q = w.q[2:3]
    check_against_decode(w, "short chain")
    # the prefix-sharing shape at 32 sequences per group: a segmented walk of
    # 511 levels, the Unshared stage first, and 4 key splits
    check_against_decode(W.make(5, 32), "prefix sweep G=32")


def test_noalloc_refuses_a_step_beyond_the_scratch():
    # 64 requests x 512 beams x 32 query heads at 100 levels: ~1.1 GB of
    # Unshared partials, far beyond the scratch; refused with no launch
    s = B.Shape(64, 512, 32, 8, 128, 64, 101, B.XATTN_BF16, 0.0)
    assert B.workspace_size(s, 100) > B.NOALLOC_SCRATCH_BYTES
    lib = B.load()
    fake = ctypes.c_void_p(0x10000)
    st = lib.xattn_decode_noalloc(ctypes.byref(s), *([fake] * 7), 100, fake, None)
    assert st == B.XATTN_EINVAL
    assert "scratch" in lib.xattn_last_error().decode()
