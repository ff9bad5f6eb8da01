"""GPU parity of li_latent_score_group (LatentIndex) and li_hs_refine (HS)
against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import TOL, check_scores, check_sets, check_topk_of_own_scores, dev

pytestmark = pytest.mark.gpu


def run_latent(x, with_scores=True, flags=li.LI_LATENT_FP16):
    sc = torch.full((x.G, max(x.n_tok, 1)), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    idx = li.li_latent_score_group(dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(x.latent, x.c_dt),
                                   dev(x.c_scale), dev(x.kv_off), int(np.diff(x.kv_off).max(initial=0)), x.k,
                                   out_scores=sc, flags=flags)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy()[:, :x.n_tok] if with_scores else None)


def rel_err(gpu, ref, mag):
    """Largest |gpu - ref| / A over the scores (A = sum_h |w_h x_h|, nonzero)."""
    mag = np.asarray(mag, np.float64)
    ok = mag > 0
    return float((np.abs(np.asarray(gpu, np.float64) - ref)[ok] / mag[ok]).max(initial=0.0))


def latent_parity(x, what, flags=li.LI_LATENT_FP16, tol=TOL):
    print(f"[latent parity] {what} B={x.B} G={x.G} Dc={x.Dc} n_tok={x.n_tok} flags={flags}", flush=True)
    gi, gs = run_latent(x, flags=flags)
    ri, rs, ra = oracle.latent_score_group(x.q, x.q_dt, x.w, x.w_dec, x.w_dt, x.latent, x.c_dt, x.c_scale, x.kv_off,
                                           x.G, x.H, x.Dh, x.Dc, x.k, c_blocks=x.c_blocks)
    print(f"[latent parity] {what}: max |err| / A = {rel_err(gs, rs, ra):.3g}", flush=True)
    check_scores(gs, rs, ra, tol=tol, what=what)
    for b in range(x.B):
        sl = slice(x.kv_off[b], x.kv_off[b + 1])
        n = int(x.kv_off[b + 1] - x.kv_off[b])
        check_topk_of_own_scores(gi[b], [gs[l, sl] for l in range(x.G)], [n] * x.G, x.k, f"{what} b={b}")
        for l in range(x.G):
            check_sets(gi[b, l], ri[b, l], rs[l, sl], ra[l, sl], n, tol=tol, what=f"{what} b={b} l={l}")


def test_latent_group_small_ragged():
    latent_parity(inputs.make_latent(301, [3000, 0, 77, 1025], G=4, k=512), "G4 Dc256")


def test_latent_group_dc128_g3_and_g5():
    latent_parity(inputs.make_latent(302, [2000, 500], G=3, Dc=128, k=256), "G3 Dc128")
    latent_parity(inputs.make_latent(303, [1500, 2100], G=5, k=300), "G5 Dc256")


def test_latent_group_fewer_heads_and_scales():
    x = inputs.make_latent(304, [1800, 650], G=2, H=48, k=200)
    x.c_scale = np.random.default_rng(5).uniform(0.5, 2.0, size=x.n_tok).astype(np.float32)
    latent_parity(x, "G2 H48 scaled")


def test_cfg4_latent_group_sampled_requests():
    """G = 4 layers over one shared latent [16 x 131072, 256] in one pass on the
    GPU; the oracle checks two of the 16 requests (all four layers) in full."""
    x = inputs.cfg4()
    print(f"[latent parity] cfg4 n_tok={x.n_tok}", flush=True)
    gi, gs = run_latent(x)
    for b in (0, 15):
        sl = slice(x.kv_off[b], x.kv_off[b + 1])
        y = inputs.Latent(q=x.q[b:b + 1], w=x.w[b:b + 1], w_dec=x.w_dec, latent=x.latent[sl], c_scale=None,
                          kv_off=np.array([0, 131072], np.int64), G=4, H=64, Dh=128, Dc=256, k=x.k)
        ri, rs, ra = oracle.latent_score_group(y.q, y.q_dt, y.w, y.w_dec, y.w_dt, y.latent, y.c_dt, None, y.kv_off,
                                               4, 64, 128, 256, x.k)
        check_scores(gs[:, sl], rs, ra, what=f"cfg4 b={b}")
        check_topk_of_own_scores(gi[b], [gs[l, sl] for l in range(4)], [131072] * 4, x.k, f"cfg4 b={b}")
        for l in range(4):
            check_sets(gi[b, l], ri[0, l], rs[l], ra[l], 131072, what=f"cfg4 b={b} l={l}")
    # Every request's selection against its own GPU scores: some of these rows
    # put over 6000 candidate keys at or above the threshold bin.
    for b in range(1, 15):
        sl = slice(x.kv_off[b], x.kv_off[b + 1])
        check_topk_of_own_scores(gi[b], [gs[l, sl] for l in range(4)], [131072] * 4, x.k, f"cfg4 b={b}")


# ---- HS ------------------------------------------------------------------------

def run_anchor(a):
    idx = li.li_index_decode(dev(a.q, "bf16"), dev(a.w), dev(a.kc, a.k_dt), dev(a.k_scale), dev(a.kv_off),
                             int(np.diff(a.kv_off).max(initial=0)), a.k)
    torch.cuda.synchronize()
    return idx


def run_followers(cand, f, with_scores=True, flags=li.LI_LATENT_FP16):
    B, C = cand.shape
    sc = torch.full((B, f.G, C), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    idx = li.li_hs_refine(cand, dev(f.q, "bf16"), dev(f.w), dev(f.w_dec, "bf16"), dev(f.latent, f.c_dt),
                          dev(f.c_scale), dev(f.kv_off), f.k, out_scores=sc, flags=flags)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy() if with_scores else None)


def hs_parity(h, what, requests=None, flags=li.LI_LATENT_FP16, tol=TOL):
    a, f = h.anchor, h.followers
    print(f"[hs parity] {what} B={a.B} C={h.C} Gf={f.G} flags={flags}", flush=True)
    cand_t = run_anchor(a)
    cand = cand_t.cpu().numpy()
    gi, gs = run_followers(cand_t, f, flags=flags)
    requests = range(a.B) if requests is None else requests
    for b in requests:
        sl = slice(a.kv_off[b], a.kv_off[b + 1])
        n = int(a.kv_off[b + 1] - a.kv_off[b])
        one = np.array([0, n], np.int64)
        # (i) the anchor: its own top-C against the oracle's
        ai, as_, aa = oracle.index_decode(a.q[b:b + 1], a.q_dt, a.w[b:b + 1], a.kc[sl], a.k_dt, a.k_scale[sl], one,
                                          a.H, a.D, h.C)
        check_sets(cand[b], ai[0], as_, aa, n, what=f"{what} anchor b={b}")
        # (ii) followers fed the GPU's candidates: scores, own-score top-k, sets
        ri, rs, ra = oracle.hs_refine(cand[b:b + 1], f.q[b:b + 1], f.q_dt, f.w[b:b + 1], f.w_dec, f.w_dt,
                                      f.latent[sl], f.c_dt, None if f.c_scale is None else f.c_scale[sl], one,
                                      f.G, f.H, f.Dh, f.Dc, f.k, c_blocks=f.c_blocks)
        nv = int((cand[b] >= 0).sum())
        print(f"[hs parity] {what} b={b}: max |err| / A = {rel_err(gs[b, :, :nv], rs[0, :, :nv], ra[0, :, :nv]):.3g}",
              flush=True)
        check_scores(gs[b, :, :nv], rs[0, :, :nv], ra[0, :, :nv], tol=tol, what=f"{what} b={b}")
        for fl in range(f.G):
            slot = oracle.topk(gs[b, fl, :nv].astype(np.float64)[None, :], [nv], f.k)[0]
            want = np.where(slot >= 0, cand[b][np.maximum(slot, 0)], -1)
            assert np.array_equal(gi[b, fl], want), f"{what} b={b} f={fl}: selection != top-k of own scores"
            # positions -> compare with the oracle's selection in slot space
            pos_s = np.full(n, np.nan)
            pos_a = np.full(n, np.nan)
            pos_s[cand[b][:nv]] = rs[0, fl, :nv]
            pos_a[cand[b][:nv]] = ra[0, fl, :nv]
            g = gi[b, fl]
            r = ri[0, fl]
            gv, rv = g[g >= 0], r[r >= 0]
            assert len(gv) == len(rv) == min(nv, f.k)
            assert np.isin(gv, cand[b][:nv]).all(), "followers must choose from the candidate set"
            diff = np.setxor1d(gv, rv)
            if diff.size:
                th = rv[np.argmin(pos_s[rv])]
                ok = np.abs(pos_s[diff] - pos_s[th]) <= tol * (pos_a[diff] + pos_a[th])
                assert ok.all(), f"{what} b={b} f={fl}: set differences beyond tolerance"


def test_hs_small():
    hs_parity(inputs.make_hs(401, [9000, 3000, 500, 0], C=4096, Gf=3, k=1024), "small")


def test_hs_candidates_equal_k_and_two_followers():
    h = inputs.make_hs(402, [5000, 2000], C=1024, Gf=2, k=1024)
    hs_parity(h, "C=k")
    cand = run_anchor(h.anchor)
    gi, _ = run_followers(cand, h.followers, with_scores=False)
    c = cand.cpu().numpy()
    for b in range(2):
        for fl in range(2):
            assert np.array_equal(gi[b, fl], c[b])


def test_cfg5_hs_sampled_requests():
    """Anchor top-8192 over 16 x 131072 fp8 keys, three latent followers
    rescoring 8192 candidates each; the oracle checks two requests in full."""
    hs_parity(inputs.cfg5(), "cfg5", requests=(0, 15))


# ---- LI_LATENT_SPLIT_BF16 ------------------------------------------------------
# The same parity checks with the absorbed query as two bf16 parts against the
# latent as stored; its scores are also held to a tighter bound than 2e-3 * A
# (the form's error measures about 2e-6 * A; the fp16 form's about 2e-4 * A).

SPLIT_TOL = 2e-5


def test_latent_group_split_bf16():
    latent_parity(inputs.make_latent(311, [3000, 0, 77, 1025], G=4, k=512), "split G4 Dc256",
                  flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)
    x = inputs.make_latent(312, [2000, 700], G=3, Dc=128, H=48, k=256)
    x.c_scale = np.random.default_rng(6).uniform(0.5, 2.0, size=x.n_tok).astype(np.float32)
    latent_parity(x, "split G3 Dc128 H48 scaled", flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)
    latent_parity(inputs.make_latent(313, [1500, 2100], G=5, k=300), "split G5 Dc256",
                  flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)


def test_hs_split_bf16():
    hs_parity(inputs.make_hs(411, [9000, 3000, 500, 0], C=4096, Gf=3, k=1024), "split",
              flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)


def test_latent_group_fp8_block_scales():
    # fp8 latent with one scale per 128 values, decoded exactly and scaled into fp16
    latent_parity(inputs.latent_to_fp8(inputs.make_latent(321, [3000, 0, 77, 1025], G=4, k=512)), "fp8 G4 Dc256")
    latent_parity(inputs.latent_to_fp8(inputs.make_latent(322, [2000, 500], G=3, Dc=128, k=256)), "fp8 G3 Dc128")


def test_hs_fp8_followers():
    h = inputs.make_hs(323, [9000, 3000, 500], C=2048, Gf=3, k=512)
    inputs.latent_to_fp8(h.followers)
    hs_parity(h, "HS fp8 followers")


def test_latent_group_fp8_long_rows():
    # rows longer than one scan segment, so the segmented top-k runs
    x = inputs.latent_to_fp8(inputs.make_latent(324, [40000, 9000], G=4, k=2048))
    latent_parity(x, "fp8 G4 L40000")


def test_latent_fp8_rejects_missing_scales_and_the_split_form():
    x = inputs.latent_to_fp8(inputs.make_latent(325, [500], G=2, k=64))
    args = (dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(x.latent, x.c_dt))
    with pytest.raises(li.LiError) as e:
        li.li_latent_score_group(*args, None, dev(x.kv_off), 500, x.k)
    assert e.value.status == li.LI_E_NULL
    with pytest.raises(li.LiError) as e:
        li.li_latent_score_group(*args, dev(x.c_scale), dev(x.kv_off), 500, x.k, flags=li.LI_LATENT_SPLIT_BF16)
    assert e.value.status == li.LI_E_UNSUPPORTED


# ---- head counts and batch sizes off the tuned shape ---------------------------

def test_latent_few_heads_run_the_split_form():
    """With 2..15 heads the default form scores a bf16 latent in the split
    form (the fp16 absorbed query's rounding nears the tolerance there): its
    scores are bit-identical to an explicit LI_LATENT_SPLIT_BF16 call."""
    for H, seed in ((2, 331), (4, 332), (8, 333), (15, 334)):
        x = inputs.make_latent(seed, [1500, 700, 33], G=2, H=H, k=128)
        latent_parity(x, f"H={H} default")
        _, s0 = run_latent(x)
        _, s1 = run_latent(x, flags=li.LI_LATENT_SPLIT_BF16)
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), f"H={H}: default form is not the split form"


def test_latent_sixteen_heads_fp16_and_fp8():
    latent_parity(inputs.make_latent(335, [2500, 900], G=3, H=16, k=256), "H=16 fp16")
    latent_parity(inputs.latent_to_fp8(inputs.make_latent(336, [2500, 900], G=3, H=16, k=256)), "H=16 fp8")


def test_latent_batches_past_one_absorption_pass():
    """B = 17 and 37: the absorption handles 16 requests per pass, so these
    run a second and a third pass with a partial tail of requests."""
    for B, seed in ((17, 341), (37, 342)):
        lens = [40 + 53 * ((7 * i) % B) for i in range(B)]
        x = inputs.make_latent(seed, lens, G=2, k=96)
        latent_parity(x, f"B={B} fp16")
        latent_parity(x, f"B={B} split", flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)


def test_hs_batches_past_one_absorption_pass_and_few_heads():
    lens = [300 + 97 * i for i in range(17)]
    h = inputs.make_hs(343, lens, C=512, Gf=2, k=128)
    hs_parity(h, "HS B=17 fp16")
    hs_parity(h, "HS B=17 split", flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)
    hs_parity(inputs.make_hs(344, [3000, 1200], C=1024, Gf=2, H=4, k=256), "HS H=4 (split form)")


def test_latent_and_hs_dc192():
    """Dc = 192 (64 rotary + 128 other dims, the shared latent of the page's
    DeepSeek-V3.2 configuration): fp16, split and fp8 (a 128-value block and a
    64-value tail block) forms, rows longer than a scan segment, and HS."""
    x = inputs.make_latent(351, [3000, 0, 77, 1025], G=4, Dc=192, k=512)
    latent_parity(x, "Dc192 fp16")
    latent_parity(x, "Dc192 split", flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)
    latent_parity(inputs.latent_to_fp8(inputs.make_latent(352, [40000, 9000], G=3, Dc=192, k=2048)), "Dc192 fp8 L40000")
    h = inputs.make_hs(353, [9000, 3000, 500], C=2048, Gf=3, Dc=192, k=512)
    hs_parity(h, "HS Dc192")
    hs_parity(h, "HS Dc192 split", flags=li.LI_LATENT_SPLIT_BF16, tol=SPLIT_TOL)
    inputs.latent_to_fp8(h.followers)
    hs_parity(h, "HS Dc192 fp8")
