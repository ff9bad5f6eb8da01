"""GPU selection step (li_topk) against the oracle's full-sort top-k on the
same fp32 scores: bit-exact indices, including ties, -0/+0 and short rows."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li

pytestmark = pytest.mark.gpu


def run(scores, k, lens=None):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).cuda()
    rl = None if lens is None else torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    out = li.li_topk(s, k, row_len=rl)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def ref(scores, k, lens=None):
    scores = np.asarray(scores, dtype=np.float32).astype(np.float64)
    lens = [scores.shape[1]] * scores.shape[0] if lens is None else lens
    return oracle.topk(scores, lens, k)


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (4096, 2048), (4097, 2048), (65536, 2048), (131072, 2048),
                                 (131072, 8192), (20000, 16384), (3000, 1), (70001, 2048)])
def test_topk_random_rows(n, k):
    rng = np.random.default_rng(n * 7 + k)
    s = rng.standard_normal((3, n)).astype(np.float32)
    print(f"[topk] n={n} k={k}", flush=True)
    assert np.array_equal(run(s, k), ref(s, k))


def test_topk_heavy_ties_and_signed_zeros():
    rng = np.random.default_rng(3)
    s = rng.integers(-3, 4, size=(4, 50000)).astype(np.float32)
    s[1] = 0.0
    s[2, ::2] = -0.0
    s[2, 1::2] = 0.0
    s[3, :] = 1.0
    s[3, 777] = 2.0
    for k in (1, 2, 1000, 2048, 16384):
        assert np.array_equal(run(s, k), ref(s, k)), k


def test_topk_ragged_rows_and_empty_rows():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((6, 9000)).astype(np.float32)
    lens = [0, 1, 2048, 2049, 8999, 9000]
    assert np.array_equal(run(s, 2048, lens), ref(s, 2048, lens))


def test_topk_extreme_values():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((2, 10000)).astype(np.float32)
    s[0, :50] = np.float32(3.4e38)
    s[0, 50:100] = np.float32(-3.4e38)
    s[1, :] = np.float32(1e-40)  # subnormal
    s[1, 5000:] = np.float32(-1e-40)
    for k in (10, 60, 2048):
        assert np.array_equal(run(s, k), ref(s, k))
