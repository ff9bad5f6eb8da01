"""Metamorphic GPU tests: relations the method fixes whatever the inputs
(IndexCache page, Symbol Map: one score per visible position, a sum over heads
of weighted ReLUs of per-head dot products).

  * head permutation: permuting the heads of q together with their weights
    (and, for the latent forms, the decoder's head blocks) leaves every score;
  * token permutation: permuting cached rows permutes the scores the same way
    and maps the selection through the permutation;
  * w -> 2 w doubles every score and keeps the selection.

On integer-valued inputs every partial sum is exact, so the relations hold bit
for bit; on float inputs the permuted call is held to the parity bar against
the oracle's scores of the unpermuted inputs, and doubling w (a power of two,
applied to every term) is still exact."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import check_scores, dev

pytestmark = pytest.mark.gpu


def int_prefill(seed, T, L, H, k):
    """Prefill inputs with integer q_hat, K_hat in [-3, 3] (exact in E4M3), integer
    w in [-2, 2] and power-of-two scales: every partial sum is an exact integer."""
    rng = np.random.default_rng(seed)
    x = inputs.make_prefill(seed, T=T, L=L, H=H, k=k)
    x.q = inputs.encode_fp8(rng.integers(-3, 4, size=(T, H, 128)).astype(np.float32))
    x.kc = inputs.encode_fp8(rng.integers(-3, 4, size=(L, 128)).astype(np.float32))
    x.w = rng.integers(-2, 3, size=(T, H)).astype(np.float32)
    x.q_scale = (2.0 ** rng.integers(-2, 3, size=T)).astype(np.float32)
    x.k_scale = (2.0 ** rng.integers(-2, 3, size=L)).astype(np.float32)
    return x


def prefill(x):
    sc = torch.full((x.T, x.L), float("nan"), dtype=torch.float32, device="cuda")
    idx = li.li_index_prefill(dev(x.q, "fp8_e4m3"), dev(x.q_scale), dev(x.w), dev(x.kc, "fp8_e4m3"),
                              dev(x.k_scale), x.qpos0, x.k, out_scores=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def test_prefill_integer_inputs_are_exact_and_metamorphic():
    x = int_prefill(601, T=24, L=1100, H=16, k=300)
    print(f"[metamorphic] prefill integer T={x.T} L={x.L} H={x.H}", flush=True)
    gi, gs = prefill(x)
    ri, rs, _ = oracle.index_prefill(x.q, x.q_dt, x.q_scale, x.w, x.kc, x.k_dt, x.k_scale, x.T, x.L, x.qpos0, x.H,
                                     x.D, x.k)
    vis = np.isfinite(rs)
    assert np.array_equal(gs[vis] + 0.0, rs[vis] + 0.0), "integer prefill scores not bit-exact"
    assert np.array_equal(gi, ri)
    # heads permuted together with their weights
    perm = np.random.default_rng(6011).permutation(x.H)
    y = int_prefill(601, T=24, L=1100, H=16, k=300)
    y.q, y.w = y.q[:, perm], y.w[:, perm]
    pi, ps = prefill(y)
    assert np.array_equal(ps.view(np.uint32), gs.view(np.uint32)) and np.array_equal(pi, gi)
    # w -> 2w
    y = int_prefill(601, T=24, L=1100, H=16, k=300)
    y.w = y.w * np.float32(2)
    di, ds = prefill(y)
    assert np.array_equal(ds[vis], 2 * gs[vis]) and np.array_equal(di, gi)
    # keys permuted inside the prefix every row sees (positions <= qpos0)
    tp = np.random.default_rng(6012).permutation(x.qpos0 + 1)
    y = int_prefill(601, T=24, L=1100, H=16, k=300)
    y.kc[:x.qpos0 + 1] = y.kc[tp]
    y.k_scale[:x.qpos0 + 1] = y.k_scale[tp]
    _, ts = prefill(y)
    assert np.array_equal(ts[:, :x.qpos0 + 1], gs[:, tp]) and np.array_equal(ts[:, x.qpos0 + 1:], gs[:, x.qpos0 + 1:])


def test_decode_integer_head_and_token_permutation():
    x = inputs.make_decode(602, [3000, 1700, 64], H=64, k=512, k_dt="bf16", dist="int")
    args = lambda z: (dev(z.q, "bf16"), dev(z.w), dev(z.kc, "bf16"), None, dev(z.kv_off), 3000, z.k)
    sc0 = torch.empty(x.n_tok, dtype=torch.float32, device="cuda")
    i0 = li.li_index_decode(*args(x), out_scores=sc0).cpu().numpy()
    s0 = sc0.cpu().numpy()
    perm = np.random.default_rng(6021).permutation(64)
    y = inputs.make_decode(602, [3000, 1700, 64], H=64, k=512, k_dt="bf16", dist="int")
    y.q, y.w = y.q[:, perm], y.w[:, perm]
    sc1 = torch.empty(x.n_tok, dtype=torch.float32, device="cuda")
    i1 = li.li_index_decode(*args(y), out_scores=sc1).cpu().numpy()
    assert np.array_equal(sc1.cpu().numpy().view(np.uint32), s0.view(np.uint32)) and np.array_equal(i1, i0)
    # request 0's rows permuted: scores follow the rows; the selection (ties
    # to the lower position) is the oracle's top-k of the permuted scores
    tp = np.random.default_rng(6022).permutation(3000)
    y = inputs.make_decode(602, [3000, 1700, 64], H=64, k=512, k_dt="bf16", dist="int")
    y.kc[:3000] = y.kc[tp]
    sc2 = torch.empty(x.n_tok, dtype=torch.float32, device="cuda")
    i2 = li.li_index_decode(*args(y), out_scores=sc2).cpu().numpy()
    s2 = sc2.cpu().numpy()
    assert np.array_equal(s2[:3000], s0[tp]) and np.array_equal(s2[3000:], s0[3000:])
    want = oracle.topk(s0[tp].astype(np.float64)[None, :], [3000], 512)[0]
    assert np.array_equal(i2[0], want) and np.array_equal(i2[1:], i0[1:])


def latent_call(x, flags=li.LI_LATENT_FP16):
    sc = torch.full((x.G, x.n_tok), float("nan"), dtype=torch.float32, device="cuda")
    idx = li.li_latent_score_group(dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(x.latent, x.c_dt),
                                   dev(x.c_scale), dev(x.kv_off), int(np.diff(x.kv_off).max()), x.k, out_scores=sc,
                                   flags=flags)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def permute_latent_heads(x, perm):
    Dh = x.Dh
    x.q, x.w = x.q[:, :, perm], x.w[:, :, perm]
    cols = (perm[:, None] * Dh + np.arange(Dh)[None, :]).reshape(-1)
    x.w_dec = np.ascontiguousarray(x.w_dec[:, :, cols])
    return x


@pytest.mark.parametrize("flags", [li.LI_LATENT_FP16, li.LI_LATENT_SPLIT_BF16])
def test_latent_metamorphic(flags):
    mk = lambda: inputs.make_latent(603, [2500, 900], G=3, k=256)
    x = mk()
    print(f"[metamorphic] latent flags={flags}", flush=True)
    gi, gs = latent_call(x, flags)
    _, rs, ra = oracle.latent_score_group(x.q, x.q_dt, x.w, x.w_dec, x.w_dt, x.latent, x.c_dt, x.c_scale, x.kv_off,
                                          x.G, x.H, x.Dh, x.Dc, x.k)
    # heads permuted with their weights and decoder blocks: within the bar of the unpermuted oracle
    y = permute_latent_heads(mk(), np.random.default_rng(6031).permutation(64))
    _, ps = latent_call(y, flags)
    check_scores(ps, rs, ra, what="latent head permutation")
    # w -> 2w: exact
    y = mk()
    y.w = y.w * np.float32(2)
    di, ds = latent_call(y, flags)
    assert np.array_equal(ds, 2 * gs) and np.array_equal(di, gi)
    # request 1's latent rows permuted: its scores follow the rows bit for bit
    tp = np.random.default_rng(6032).permutation(900)
    y = mk()
    y.latent[2500:] = y.latent[2500 + tp]
    ti, ts = latent_call(y, flags)
    assert np.array_equal(ts[:, 2500:], gs[:, 2500 + tp]) and np.array_equal(ts[:, :2500], gs[:, :2500])
    for l in range(3):
        want = oracle.topk(gs[l, 2500 + tp].astype(np.float64)[None, :], [900], 256)[0]
        assert np.array_equal(ti[1, l], want)


def test_hs_metamorphic():
    mk = lambda: inputs.make_hs(604, [4000, 1500], C=1024, Gf=2, k=256)
    h = mk()
    a, f = h.anchor, h.followers
    cand = li.li_index_decode(dev(a.q, "bf16"), dev(a.w), dev(a.kc, a.k_dt), dev(a.k_scale), dev(a.kv_off), 4000,
                              h.C)

    def follow(fx):
        sc = torch.full((2, fx.G, h.C), float("nan"), dtype=torch.float32, device="cuda")
        idx = li.li_hs_refine(cand, dev(fx.q, "bf16"), dev(fx.w), dev(fx.w_dec, "bf16"), dev(fx.latent, fx.c_dt),
                              None, dev(fx.kv_off), fx.k, out_scores=sc)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), sc.cpu().numpy()
    gi, gs = follow(f)
    c = cand.cpu().numpy()
    # w -> 2w: exact
    g2 = mk().followers
    g2.w = g2.w * np.float32(2)
    di, ds = follow(g2)
    nv = [(c[b] >= 0).sum() for b in range(2)]
    for b in range(2):
        assert np.array_equal(ds[b, :, :nv[b]], 2 * gs[b, :, :nv[b]])
    assert np.array_equal(di, gi)
    # heads permuted: within the bar of the oracle's unpermuted scores
    p = permute_latent_heads(mk().followers, np.random.default_rng(6041).permutation(64))
    _, ps = follow(p)
    for b in range(2):
        sl = slice(f.kv_off[b], f.kv_off[b + 1])
        one = np.array([0, f.kv_off[b + 1] - f.kv_off[b]], np.int64)
        _, rs, ra = oracle.hs_refine(c[b:b + 1], f.q[b:b + 1], f.q_dt, f.w[b:b + 1], f.w_dec, f.w_dt, f.latent[sl],
                                     f.c_dt, None, one, f.G, f.H, f.Dh, f.Dc, f.k)
        check_scores(ps[b, :, :nv[b]], rs[0, :, :nv[b]], ra[0, :, :nv[b]], what=f"HS head permutation b={b}")
