"""The measurement aids: li_read_probe reads every word it is given, and
li_mfma_probe runs the products it reports (constant operands give exact
sums) and records a plausible shader clock."""
import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as li

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1 << 20, (1 << 22) + 48])
def test_read_probe_folds_every_word(nbytes):
    g = np.random.default_rng(nbytes)
    words = g.integers(-(1 << 31), 1 << 31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words).cuda()
    sink = torch.zeros(li.LI_READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    li.li_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words.view(np.uint32))
    assert got == want


@pytest.mark.parametrize("form,K", [(li.LI_MFMA_PROBE_F16, 32), (li.LI_MFMA_PROBE_BF16, 16),
                                    (li.LI_MFMA_PROBE_FP8, 128)])
def test_mfma_probe_constant_operands_sum_exactly(form, K):
    iters = 64
    sink = torch.full((li.LI_MFMA_PROBE_SINK_WORDS,), -1.0, dtype=torch.float32, device="cuda")
    clk = torch.zeros(li.LI_MFMA_PROBE_CLOCK_WORDS, dtype=torch.int32, device="cuda")
    li.li_mfma_probe(form, False, iters, sink, clk)
    torch.cuda.synchronize()
    # two chains of eight products per iteration, each adding K to every accumulator element
    assert np.all(sink.cpu().numpy() == 2 * 8 * K * iters)
    c = clk.cpu().numpy().view(np.uint32).astype(np.float64).reshape(-1, 2)
    assert np.all(c[:, 0] > 0) and np.all(c[:, 1] > 0)
    mhz = c[:, 0].sum() / c[:, 1].sum() * 100.0
    assert 300.0 < mhz < 3500.0


@pytest.mark.parametrize("form", [li.LI_MFMA_PROBE_F16, li.LI_MFMA_PROBE_BF16, li.LI_MFMA_PROBE_FP8])
def test_mfma_probe_random_operands_stay_finite(form):
    sink = torch.zeros(li.LI_MFMA_PROBE_SINK_WORDS, dtype=torch.float32, device="cuda")
    clk = torch.zeros(li.LI_MFMA_PROBE_CLOCK_WORDS, dtype=torch.int32, device="cuda")
    li.li_mfma_probe(form, True, 64, sink, clk)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.all(np.isfinite(s))
    assert len(np.unique(s)) > s.size // 2  # waves saw different operands
