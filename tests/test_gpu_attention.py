"""GPU parity of li_sparse_attention against the CPU oracle.

Scores accumulate in fp32 and each weight p is rounded to bf16 before the
value product (and its sum), so every weight carries a relative error of at
most 2^-9 and |o_gpu - o_ref| <= 2 * 2^-9 * mag, mag = sum_j p_j |v_j| / sum_j p_j
(the oracle's error scale); the bar below is 5e-3 * mag + 1e-6.  A single
selected token and a zero query have exact answers (the value row, the mean of
the values) and are checked to fp32 rounding."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import dev

pytestmark = pytest.mark.gpu

TOL = 5e-3


def run(x, kv=None, q=None):
    kv = dev(x.kv, "bf16") if kv is None else kv
    out = li.li_sparse_attention(dev(x.q if q is None else q, "bf16"), kv, dev(x.idx), dev(x.kv_off), x.scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, ref, mag, what, tol=TOL):
    err = np.abs(got - ref)
    rel = float((err / (mag + 1e-30)).max(initial=0.0))
    print(f"[attention parity] {what}: max |err| / mag = {rel:.3g}", flush=True)
    assert np.all(err <= tol * mag + 1e-6), f"{what}: max |err|/mag {rel:.3g}"


def parity(x, what):
    print(f"[attention parity] {what} B={x.B} H={x.H} k={x.k} n_tok={x.n_tok}", flush=True)
    got = run(x)
    ref, mag = oracle.sparse_attention(x.q, "bf16", x.kv, "bf16", x.idx, x.kv_off, x.scale, 512)
    check(got, ref, mag, what)


def test_attention_small_ragged_h64():
    parity(inputs.make_attention(501, [5000, 100, 3000], H=64, k=256), "H64 k256 ragged")


def test_attention_h128_k2048_with_short_and_empty_requests():
    parity(inputs.make_attention(502, [9000, 700, 0, 4100], H=128, k=2048), "H128 k2048 short+empty")


def test_attention_k_not_a_multiple_of_the_tile():
    parity(inputs.make_attention(503, [400, 90], H=64, k=100), "H64 k100")
    parity(inputs.make_attention(504, [33], H=192, k=33), "H192 k33")


def test_attention_single_selected_token_returns_its_value_row():
    x = inputs.make_attention(505, [300, 50], H=64, k=64)
    x.idx[:, 1:] = -1
    got = run(x)
    kvv = torch.from_numpy(x.kv.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(x.B):
        v = kvv[x.kv_off[b] + x.idx[b, 0], :512]
        assert np.array_equal(got[b], np.broadcast_to(v, got[b].shape)), f"request {b}"


def test_attention_zero_query_is_the_mean_of_the_values():
    x = inputs.make_attention(506, [3000, 2100], H=64, k=2048)
    q0 = np.zeros_like(x.q)
    got = run(x, q=q0)
    kvv = torch.from_numpy(x.kv.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(x.B):
        sel = x.idx[b][x.idx[b] >= 0]
        mean = kvv[x.kv_off[b] + sel, :512].mean(axis=0)
        assert np.allclose(got[b], mean[None, :], rtol=0, atol=1e-5)


def test_attention_full_decode_step_sampled():
    x = inputs.attention_decode()
    kv = inputs.device_kv_cache(x)
    got = run(x, kv=kv)
    rng = np.random.default_rng(507)
    for b in rng.choice(x.B, 4, replace=False):
        rows = torch.from_numpy(x.kv_off[b] + x.idx[b].astype(np.int64)).cuda()
        sub = kv.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)
        heads = rng.choice(x.H, 8, replace=False)
        ref, mag = oracle.sparse_attention(x.q[b:b + 1, heads], "bf16", sub, "bf16",
                                           np.arange(x.k, dtype=np.int32)[None], np.array([0, x.k], np.int64),
                                           x.scale, 512)
        check(got[b, heads][None], ref, mag, f"{x.name} b={b}")


def test_attention_ignores_workspace_contents():
    x = inputs.make_attention(508, [2500, 1800, 600], H=128, k=512)
    first = run(x)
    need = li.lib().li_sparse_attention_ws(x.B, x.H, x.k)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    out = li.li_sparse_attention(dev(x.q, "bf16"), dev(x.kv, "bf16"), dev(x.idx), dev(x.kv_off), x.scale, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), first)
