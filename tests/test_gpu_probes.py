"""The measurement probes behind the benchmark's achievable-peak leg.

xattn_peak_read must visit every 16-byte unit of its buffer exactly once:
the XOR of the per-thread words it writes equals the XOR of all the
buffer's words (ragged sizes leave a tail that the last loop covers).
xattn_peak_mfma_bf16 reports the operations it performs and writes the same
finite values on every run.
"""
import numpy as np
import pytest
import torch

from generative_recommendation_beam_xattn_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,blocks", [(4, 1), (4 * 1000 + 4 * 7, 3), (1 << 20, 64),
                                             (4 * 777777, 2048)])
def test_peak_read_visits_every_unit_once(n_words, blocks):
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 31 - 1, size=n_words, dtype=np.int32)
    src = torch.from_numpy(host).cuda()
    out = B.peak_read(src, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)


def test_peak_mfma_counts_and_repeats():
    f1, o1 = B.peak_mfma_bf16(10, 8)
    f2, o2 = B.peak_mfma_bf16(10, 8)
    torch.cuda.synchronize()
    assert f1 == f2 == 8 * 4 * 10 * 4 * 2 * 32 * 32 * 16
    assert torch.isfinite(o1).all() and torch.equal(o1, o2)


def test_probe_arguments_rejected():
    src = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(B.XattnError):
        B.peak_read(src[:3], 4)       # 12 bytes: not a multiple of 16
    with pytest.raises(B.XattnError):
        B.peak_mfma_bf16(0, 4)
