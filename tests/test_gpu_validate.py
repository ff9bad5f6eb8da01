"""LI_DEBUG_VALIDATE: with the variable set, each entry point checks its device
inputs' preconditions first and reports the first violation as LI_E_VALUE;
valid inputs give the same results as without it.  Every bad input here is
rejected before any scan or selection kernel runs."""
import os

import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def validating():
    old = os.environ.get("LI_DEBUG_VALIDATE")
    os.environ["LI_DEBUG_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["LI_DEBUG_VALIDATE"]
    else:
        os.environ["LI_DEBUG_VALIDATE"] = old


def rejected(fn, text):
    with pytest.raises(li.LiError) as e:
        fn()
    assert e.value.status == li.LI_E_VALUE, e.value
    assert text in str(e.value), e.value
    print(f"[validate] rejected: {e.value}", flush=True)


def decode_args(x):
    return [dev(x.q, "bf16"), dev(x.w), dev(x.kc, x.k_dt), dev(x.k_scale), dev(x.kv_off),
            int(x.lens.max(initial=0)), x.k]


def test_decode_checks(validating):
    x = inputs.make_decode(701, [3000, 1200], k=256)
    print("[validate] decode valid", flush=True)
    good = li.li_index_decode(*decode_args(x))
    os.environ["LI_DEBUG_VALIDATE"] = "0"
    plain = li.li_index_decode(*decode_args(x))
    os.environ["LI_DEBUG_VALIDATE"] = "1"
    torch.cuda.synchronize()
    assert torch.equal(good, plain)

    a = decode_args(x)
    a[4] = dev(np.array([0, 3000, 2999], np.int64))
    rejected(lambda: li.li_index_decode(*a), "kv_off decreases")
    a = decode_args(x)
    a[4] = dev(np.array([0, 3000, 4300], np.int64))
    rejected(lambda: li.li_index_decode(*a), "outside [0, n_tok]")
    a = decode_args(x)
    a[5] = 2000
    rejected(lambda: li.li_index_decode(*a), "longer than max_len")
    ks = x.k_scale.copy()
    ks[1234] = 0.0
    a = decode_args(x)
    a[3] = dev(ks)
    rejected(lambda: li.li_index_decode(*a), "k_scale")
    kc = x.kc.copy()
    kc[77, 5] = 0xFF
    a = decode_args(x)
    a[2] = dev(kc, "fp8_e4m3")
    rejected(lambda: li.li_index_decode(*a), "k_cache")
    w = x.w.copy()
    w[1, 3] = np.inf
    a = decode_args(x)
    a[1] = dev(w)
    rejected(lambda: li.li_index_decode(*a), "w not finite")


def test_prefill_checks(validating):
    x = inputs.make_prefill(702, 40, 3000, k=128)
    args = lambda qs: (dev(x.q, "fp8_e4m3"), dev(qs), dev(x.w), dev(x.kc, "fp8_e4m3"), dev(x.k_scale), x.qpos0, x.k)
    print("[validate] prefill valid", flush=True)
    li.li_index_prefill(*args(x.q_scale))
    qs = x.q_scale.copy()
    qs[7] = -1.0
    rejected(lambda: li.li_index_prefill(*args(qs)), "q_scale")


def test_latent_and_hs_checks(validating):
    x = inputs.make_latent(703, [900, 400], G=2, k=128)
    args = lambda lat: (dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(lat, "bf16"), None, dev(x.kv_off),
                        900, x.k)
    print("[validate] latent valid", flush=True)
    li.li_latent_score_group(*args(x.latent))
    lat = x.latent.copy()
    lat[333, 9] = 0x7FC0  # bf16 NaN
    rejected(lambda: li.li_latent_score_group(*args(lat)), "latent")

    cand = np.full((2, 64), -1, np.int32)
    cand[0, :50] = np.arange(50) * 3
    cand[1, :10] = np.arange(10) * 7
    hs = lambda c: li.li_hs_refine(dev(c), dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"),
                                   dev(x.latent, "bf16"), None, dev(x.kv_off), 16)
    print("[validate] hs valid", flush=True)
    hs(cand)
    bad = cand.copy()
    bad[0, 10], bad[0, 11] = bad[0, 11], bad[0, 10]
    rejected(lambda: hs(bad), "not ascending")
    bad = cand.copy()
    bad[1, 9] = 400  # the row's last valid entry, so the order still holds
    rejected(lambda: hs(bad), "outside [-1, L_b)")
    bad = cand.copy()
    bad[1, 20] = 5
    rejected(lambda: hs(bad), "not ascending")


def test_hs_latent_rows_and_fp16_range_checks(validating):
    """The HS call checks the latent rows its candidates name (codes, scales);
    the fp16 form also checks that the latent fits fp16's range."""
    x = inputs.make_latent(705, [900, 400], G=2, H=16, k=64)
    cand = np.full((2, 64), -1, np.int32)
    cand[0, :50] = np.arange(50) * 3
    cand[1, :10] = np.arange(10) * 7

    def hs(lat, c_scale=None, c_dt="bf16", flags=li.LI_LATENT_FP16):
        return li.li_hs_refine(dev(cand), dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(lat, c_dt),
                               dev(c_scale), dev(x.kv_off), 16, flags=flags)
    print("[validate] hs latent rows", flush=True)
    hs(x.latent)
    lat = x.latent.copy()
    lat[900 + 63, 100] = 0x7F80  # +Inf in request 1's candidate row 63
    rejected(lambda: hs(lat), "latent holds")
    lat = x.latent.copy()
    lat[900 + 64, 100] = 0x7F80  # a row no candidate names is not read
    hs(lat)
    lat = x.latent.copy()
    lat[3 * 17, 5] = 0x4780  # bf16 65536: past fp16's range
    rejected(lambda: hs(lat), "fp16 range")
    hs(lat, flags=li.LI_LATENT_SPLIT_BF16)  # the split form takes any bf16 latent
    rejected(lambda: li.li_latent_score_group(dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(lat, "bf16"),
                                              None, dev(x.kv_off), 900, x.k), "fp16 range")

    y = inputs.latent_to_fp8(inputs.make_latent(706, [900, 400], G=2, H=16, k=64))
    print("[validate] hs fp8 latent rows", flush=True)
    hs(y.latent, y.c_scale, "fp8_e4m3")
    sc = y.c_scale.copy()
    sc[900 + 7 * 9, 1] = 0.0  # request 1's candidate 9, second block
    rejected(lambda: hs(y.latent, sc, "fp8_e4m3"), "c_scale not finite")
    sc = y.c_scale.copy()
    sc[3 * 2, 0] = 200.0  # 448 * 200 is past fp16's range
    rejected(lambda: hs(y.latent, sc, "fp8_e4m3"), "65504 / 448")
    rejected(lambda: li.li_latent_score_group(dev(y.q, "bf16"), dev(y.w), dev(y.w_dec, "bf16"),
                                              dev(y.latent, "fp8_e4m3"), dev(sc), dev(y.kv_off), 900, y.k),
             "65504 / 448")
    lat8 = y.latent.copy()
    lat8[3 * 4, 200] = 0x7F
    rejected(lambda: hs(lat8, y.c_scale, "fp8_e4m3"), "latent holds")


def test_topk_checks(validating):
    s = np.random.default_rng(704).standard_normal((3, 500)).astype(np.float32)
    s[0, 10] = -np.inf
    print("[validate] topk valid", flush=True)
    li.li_topk(dev(s), 20)
    s[2, 499] = np.nan
    rejected(lambda: li.li_topk(dev(s), 20), "NaN")
    rl = np.array([500, 300, 501], np.int32)
    rejected(lambda: li.li_topk(dev(s), 20, row_len=dev(rl)), "row_len")
