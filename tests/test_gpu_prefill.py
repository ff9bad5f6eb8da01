"""GPU parity of li_index_prefill (causal fp8 scan + top-k) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import check_scores, check_sets, check_topk_of_own_scores, dev

pytestmark = pytest.mark.gpu


def run_gpu(x, with_scores=True):
    sc = torch.full((x.T, x.L), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    idx = li.li_index_prefill(dev(x.q, "fp8_e4m3"), dev(x.q_scale), dev(x.w), dev(x.kc, "fp8_e4m3"),
                              dev(x.k_scale), x.qpos0, x.k, out_scores=sc)
    torch.cuda.synchronize()
    return idx, sc


def parity_rows(x, gi, gs, rows, what):
    """Full parity of the given rows; returns the largest |err| / A seen."""
    worst = 0.0
    for t in rows:
        vis = x.qpos0 + t + 1
        ri, rs, ra = oracle.index_prefill(x.q[t:t + 1], x.q_dt, x.q_scale[t:t + 1], x.w[t:t + 1], x.kc, x.k_dt,
                                          x.k_scale, 1, x.L, x.qpos0 + t, x.H, x.D, x.k)
        g = gs[t]
        assert np.isneginf(g[vis:]).all(), f"{what} t={t}: masked positions must be -inf"
        worst = max(worst, check_scores(g[:vis], rs[0, :vis], ra[0, :vis], what=f"{what} t={t}"))
        check_topk_of_own_scores(gi[t:t + 1], [g], [vis], x.k, f"{what} t={t}")
        check_sets(gi[t], ri[0], rs[0], ra[0], vis, what=f"{what} t={t}")
        assert gi[t].max() <= x.qpos0 + t
    print(f"[prefill parity] {what}: max |err| / A = {worst:.3g}", flush=True)
    return worst


def test_prefill_small_all_rows():
    x = inputs.make_prefill(201, T=37, L=1000, k=300)
    print(f"[prefill parity] T={x.T} L={x.L} qpos0={x.qpos0}", flush=True)
    gi, gs = run_gpu(x)
    parity_rows(x, gi.cpu().numpy(), gs.cpu().numpy(), range(x.T), "small")


def test_prefill_rows_shorter_than_k():
    x = inputs.make_prefill(202, T=9, L=70, k=64)
    gi, gs = run_gpu(x)
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    parity_rows(x, gi, gs, range(x.T), "short")
    assert gi[0].tolist() == list(range(62)) + [-1, -1]


def test_prefill_chunk_not_at_the_end_and_few_heads():
    x = inputs.make_prefill(203, T=20, L=600, H=24, k=128, qpos0=300)
    gi, gs = run_gpu(x)
    parity_rows(x, gi.cpu().numpy(), gs.cpu().numpy(), range(x.T), "mid-chunk H=24")


def test_prefill_eight_heads_random_and_spread_queries():
    """The fewest heads the fp8 path takes: N(0,1) queries, and queries whose
    elements spread over 2^-9 .. 2^3 inside each head (the analogue of the
    decode's spread-query test within E4M3's range), all rows checked.  The
    largest |err| / A is printed (run with -s): the figures the header quotes
    for H = 8 and H = 64 come from this test and from the small all-rows case."""
    x = inputs.make_prefill(206, T=40, L=1500, H=8, k=256)
    gi, gs = run_gpu(x)
    parity_rows(x, gi.cpu().numpy(), gs.cpu().numpy(), range(x.T), "H=8")
    x = inputs.make_prefill(207, T=40, L=1500, H=8, k=256)
    octave = 2.0 ** (3 - (np.arange(128) % 13))
    x.q = inputs.encode_fp8((np.random.default_rng(2071).standard_normal((x.T, 8, 128)) * octave).astype(np.float32))
    gi, gs = run_gpu(x)
    parity_rows(x, gi.cpu().numpy(), gs.cpu().numpy(), range(x.T), "H=8 spread q")


def test_prefill_rejects_fewer_than_eight_heads():
    x = inputs.make_prefill(208, T=4, L=100, H=4, k=16)
    with pytest.raises(li.LiError) as e:
        run_gpu(x)
    assert e.value.status == li.LI_E_UNSUPPORTED


def test_prefill_without_score_output_matches():
    x = inputs.make_prefill(204, T=16, L=3000, k=2048)
    i0, _ = run_gpu(x)
    i1, _ = run_gpu(x, with_scores=False)
    assert torch.equal(i0, i1)


def test_cfg3_prefill_sampled_rows():
    """T = 4096 new tokens against a causal L = 65536 cache on the GPU; the
    oracle checks sampled rows in full (first, last, around powers of two)."""
    x = inputs.cfg3()
    print(f"[prefill parity] cfg3 T={x.T} L={x.L}", flush=True)
    gi, gs = run_gpu(x)
    rows = [0, 1, 2047, 4094, 4095, 1234]
    sel = torch.tensor(rows, device="cuda")
    gi_np = gi.cpu().numpy()
    gsub = gs.index_select(0, sel).cpu().numpy()
    for j, t in enumerate(rows):
        vis = x.qpos0 + t + 1
        ri, rs, ra = oracle.index_prefill(x.q[t:t + 1], x.q_dt, x.q_scale[t:t + 1], x.w[t:t + 1], x.kc, x.k_dt,
                                          x.k_scale, 1, x.L, x.qpos0 + t, x.H, x.D, x.k)
        g = gsub[j]
        assert np.isneginf(g[vis:]).all()
        check_scores(g[:vis], rs[0, :vis], ra[0, :vis], what=f"cfg3 t={t}")
        check_topk_of_own_scores(gi_np[t:t + 1], [g], [vis], x.k, f"cfg3 t={t}")
        check_sets(gi_np[t], ri[0], rs[0], ra[0], vis, what=f"cfg3 t={t}")
    # every row: sizes, order, causal bound
    assert (gi_np >= 0).all()
    assert np.all(np.diff(gi_np, axis=1) > 0)
    assert np.all(gi_np.max(axis=1) <= x.qpos0 + np.arange(x.T))


def test_prefill_all_equal_scores_overflow_a_histogram_bin():
    # Zero head weights make every visible score 0, so one level-0 bin holds
    # every visible key; rows with more than 65535 of them exceed the scan's
    # 16-bit bin counters and must take the selection's own-histogram path.
    # With all scores tied the lowest positions win.
    x = inputs.make_prefill(205, T=3, L=65600, k=2048)
    x.w[:] = 0.0
    print(f"[prefill parity] tied scores T={x.T} L={x.L} qpos0={x.qpos0}", flush=True)
    gi, gs = run_gpu(x)
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    for t in range(x.T):
        vis = x.qpos0 + t + 1
        assert vis > 65535
        assert (gs[t, :vis] == 0.0).all() and np.isneginf(gs[t, vis:]).all()
        ri, _, _ = oracle.index_prefill(x.q[t:t + 1], x.q_dt, x.q_scale[t:t + 1], x.w[t:t + 1], x.kc, x.k_dt,
                                        x.k_scale, 1, x.L, x.qpos0 + t, x.H, x.D, x.k, want_scores=False)
        assert np.array_equal(gi[t], ri[0]) and np.array_equal(ri[0], np.arange(x.k, dtype=np.int32))
    # the same rows without a score output (the selection reads only the lists)
    gi2, _ = run_gpu(x, with_scores=False)
    assert np.array_equal(gi2.cpu().numpy(), gi)


def test_cfg3_every_row_selects_the_top_k_of_its_own_scores():
    """All 4096 rows of the T = 4096, L = 65536 chunk: the selection (read from
    the scan's candidate lists, whose floors rise several times per row) is
    exactly the top k of the scores the scan wrote, with ties going to the
    lowest positions; without a score output the indices are the same."""
    x = inputs.cfg3()
    print(f"[prefill parity] cfg3 every row T={x.T} L={x.L}", flush=True)
    gi, gs = run_gpu(x)
    assert x.qpos0 + 1 > x.k  # every row has more than k visible keys
    gil = gi.long()
    assert bool((gi >= 0).all()) and bool((gil.diff(dim=1) > 0).all())
    kth = gs.gather(1, gil).min(dim=1).values
    rest = gs.clone()
    rest.scatter_(1, gil, float("-inf"))
    top_rest = rest.max(dim=1).values
    assert bool((kth >= top_rest).all()), "a key above a selected one was left out"
    tied = torch.nonzero(kth == top_rest).flatten().tolist()
    for t in tied:
        g = gs[t].cpu().numpy()
        sel = gi[t].cpu().numpy()
        v = kth[t].item()
        in_sel = sel[g[sel] == v]
        out = np.setdiff1d(np.nonzero(g == v)[0], sel)
        assert out.min() > in_sel.max(), f"row {t}: a tie went to a higher position"
    print(f"[prefill parity] cfg3 every row: {len(tied)} rows with ties at the threshold", flush=True)
    del rest, gs
    gi2, _ = run_gpu(x, with_scores=False)
    assert torch.equal(gi, gi2)
