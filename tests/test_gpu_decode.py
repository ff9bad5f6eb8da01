"""GPU parity of li_index_decode (decode scan + top-k) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import check_scores, check_sets, check_topk_of_own_scores, dev

pytestmark = pytest.mark.gpu


def run_gpu(x, k=None, with_scores=True):
    k = x.k if k is None else k
    sc = torch.full((max(x.n_tok, 1),), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    idx = li.li_index_decode(dev(x.q, "bf16"), dev(x.w), dev(x.kc, x.k_dt), dev(x.k_scale), dev(x.kv_off),
                             int(x.lens.max(initial=0)), k, out_scores=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy()[:x.n_tok] if with_scores else None)


def parity(x, exact=False, what=""):
    print(f"[decode parity] {what} B={x.B} n_tok={x.n_tok} k_dt={x.k_dt} k={x.k}", flush=True)
    gi, gs = run_gpu(x)
    ri, rs, ra = oracle.index_decode(x.q, x.q_dt, x.w, x.kc, x.k_dt, x.k_scale, x.kv_off, x.H, x.D, x.k)
    check_scores(gs, rs, ra, exact=exact, what=what)
    if exact:
        assert np.array_equal(gi, ri), f"{what}: indices not bit-exact"
        return
    lens = x.lens
    rows = [gs[x.kv_off[b]:x.kv_off[b + 1]] for b in range(x.B)]
    check_topk_of_own_scores(gi, rows, lens, x.k, what)
    for b in range(x.B):
        sl = slice(x.kv_off[b], x.kv_off[b + 1])
        check_sets(gi[b], ri[b], rs[sl], ra[sl], int(lens[b]), what=f"{what} b={b}")


def test_cfg1_integer_decode_is_bit_exact():
    """Single decode query, L = 4096, integer-valued bf16: scores and indices bit-exact."""
    parity(inputs.cfg1(), exact=True, what="cfg1")


def test_integer_decode_ragged_bit_exact():
    x = inputs.make_decode(101, [1, 33, 0, 4095, 2049, 97], H=64, D=128, k=2048, k_dt="bf16", dist="int")
    parity(x, exact=True, what="int ragged")
    x = inputs.make_decode(102, [300, 31], H=64, D=128, k=1, k_dt="bf16", dist="int")
    parity(x, exact=True, what="int k=1")


def test_fp8_decode_ragged_small():
    x = inputs.make_decode(103, [5000, 0, 1, 31, 2047, 2048, 2049, 7777], k=2048)
    parity(x, what="fp8 ragged")


def test_bf16_float_decode_and_fewer_heads():
    x = inputs.make_decode(104, [3000, 1234], k=256, k_dt="bf16")
    parity(x, what="bf16 float")
    x = inputs.make_decode(105, [2500, 900], H=40, k=300)
    parity(x, what="fp8 H=40")
    x = inputs.make_decode(106, [700], H=1, k=64)
    parity(x, what="fp8 H=1")


def test_cfg2_batched_ragged_decode():
    """B = 32 requests, L_b ~ U{8192..32768}, fp8 keys with per-token scales."""
    parity(inputs.cfg2(), what="cfg2")


def test_fp8_conversion_covers_every_code():
    """Keys holding each of the 254 finite E4M3FN codes, read through q = +e_0
    (w = +1) and q = -e_0 (w = -1): the two scores are max(k, 0) and min(k, 0),
    so the GPU must reproduce the exact decoded value of every code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    n = codes.size
    kc = np.repeat(codes[:, None], 128, axis=1)
    kc = np.concatenate([kc, kc])
    q = np.zeros((2, 1, 128), np.float32)
    q[0, 0, 0], q[1, 0, 0] = 1.0, -1.0
    x = inputs.Decode(q=inputs.encode_bf16(q), w=np.array([[1.0], [-1.0]], np.float32), kc=kc, k_scale=None,
                      kv_off=np.array([0, n, 2 * n], np.int64), H=1, D=128, k=4)
    _, gs = run_gpu(x)
    dec = oracle.decode_element(codes, "fp8_e4m3")
    assert np.array_equal(gs[:n] + gs[n:], dec)


def test_fp8_decode_query_spanning_many_octaves():
    """fp8 keys against query rows whose elements span 2^0 .. 2^-30 inside each
    head and whose heads differ by up to 2^40 in size.  The scan converts each
    fp8 key to bf16 exactly and runs the bf16 product chain, so the scores meet
    the tolerance however the query's magnitudes spread, with one head too."""
    x = inputs.make_decode(111, [3000, 1500, 40], k=256)
    rng = np.random.default_rng(1111)
    octave = 2.0 ** -(np.arange(128) % 31)
    head = 2.0 ** (20.0 * (np.arange(64) % 3) - 20.0)
    q = rng.standard_normal((x.B, 64, 128)) * octave[None, None, :] * head[None, :, None]
    x.q = inputs.encode_bf16(q.astype(np.float32))
    parity(x, what="fp8 q octaves")
    x1 = inputs.make_decode(112, [2000], H=1, k=64)
    x1.q = inputs.encode_bf16((rng.standard_normal((1, 1, 128)) * octave[None, None, :]).astype(np.float32))
    parity(x1, what="fp8 q octaves H=1")


def test_decode_scale_doubling_and_determinism():
    x = inputs.make_decode(107, [6000, 4100], k=512)
    i0, s0 = run_gpu(x)
    i1, s1 = run_gpu(x)
    assert np.array_equal(i0, i1) and np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    x.k_scale = x.k_scale * np.float32(2)
    i2, s2 = run_gpu(x)
    assert np.array_equal(s2, 2 * s0) and np.array_equal(i2, i0)


def test_decode_without_score_output_matches():
    x = inputs.make_decode(108, [9000, 3000], k=2048)
    i0, _ = run_gpu(x)
    i1, _ = run_gpu(x, with_scores=False)
    assert np.array_equal(i0, i1)


def test_decode_all_equal_scores_take_the_lowest_positions():
    """w = 0 makes every score +0: the selection is positions 0 .. k-1.  Rows
    whose candidate sets exceed the final step's register capacity (8192 keys)
    and, for k = 4096, its LDS capacity (16384) take the slower paths."""
    for seed, lens, k in ((109, [20000, 12000, 8192, 70000], 2048), (110, [12000, 30000, 4096], 4096)):
        x = inputs.make_decode(seed, lens, k=k)
        x.w = np.zeros_like(x.w)
        parity(x, exact=True, what=f"all-equal k={k}")
        gi, _ = run_gpu(x)
        for b, n in enumerate(lens):
            assert np.array_equal(gi[b], np.arange(min(n, k), dtype=np.int32)), f"all-equal k={k} b={b}"


def test_decode_128k_sampled_requests():
    """The decode sweep's headline point (B = 32, L = 131072, fp8) on the GPU;
    the oracle checks two of the requests in full."""
    x = inputs.decode_sweep(131072)
    print(f"[decode parity] sweep L=131072 B={x.B}", flush=True)
    gi, gs = run_gpu(x)
    for b in (0, 31):
        sl = slice(x.kv_off[b], x.kv_off[b + 1])
        y = inputs.Decode(q=x.q[b:b + 1], w=x.w[b:b + 1], kc=x.kc[sl], k_scale=x.k_scale[sl],
                          kv_off=np.array([0, 131072], np.int64), H=64, D=128, k=x.k)
        ri, rs, ra = oracle.index_decode(y.q, y.q_dt, y.w, y.kc, y.k_dt, y.k_scale, y.kv_off, 64, 128, x.k)
        check_scores(gs[sl], rs, ra, what=f"128K b={b}")
        check_topk_of_own_scores(gi[b:b + 1], [gs[sl]], [131072], x.k, f"128K b={b}")
        check_sets(gi[b], ri[0], rs, ra, 131072, what=f"128K b={b}")


def test_decode_largest_k():
    """k = LI_MAX_K (16384): the top-k's final step holds the candidates in
    dynamic LDS; with w = 0 (every score +0) the candidates exceed that and
    the step runs from global memory."""
    x = inputs.make_decode(111, [40000, 16384, 16385, 70000, 5], k=li.LI_MAX_K)
    parity(x, what="k=16384")
    x.w = np.zeros_like(x.w)
    parity(x, exact=True, what="k=16384 all-equal")


def test_decode_many_short_requests():
    """A batch of 300 short requests (0 .. 400 keys) with k = 64: many rows
    keep all their keys, the rest select from a few hundred."""
    lens = np.random.default_rng(112).integers(0, 401, size=300)
    parity(inputs.make_decode(112, lens.tolist(), k=64), what="B=300 short")


def test_decode_bucket_selection_ties_and_capacity():
    """Rows of at most 32 scan workgroups of at least 2k keys select from the
    scan's bin-ordered candidate lists (one workgroup per row); here k = 256
    and 512 keys per scan workgroup.  With w = 0 every key ties at +0, so the
    whole row is the threshold bin and goes through both radix levels; the
    lowest positions win."""
    lens = [5000, 3000, 16384, 257, 256, 0, 9000]
    x = inputs.make_decode(113, lens, k=256)
    parity(x, what="bucket random")
    x.w = np.zeros_like(x.w)
    parity(x, exact=True, what="bucket all-equal")
    gi, _ = run_gpu(x, with_scores=False)
    for b, n in enumerate(lens):
        want = np.concatenate([np.arange(min(n, 256)), -np.ones(256 - min(n, 256))]).astype(np.int32)
        assert np.array_equal(gi[b], want), f"bucket all-equal b={b}"


def test_decode_128k_every_row_selects_the_top_k_of_its_own_scores():
    """B = 32 requests of 131072 fp8 keys, k = 2048 (bucket selection, 16 scan
    workgroups per row): every row's indices are the top k of the scores the
    scan wrote, ties to the lowest positions, and the same without a score
    output.  With w = 0 (all scores +0) the candidate sets are whole rows,
    read from global memory, and the selection is positions 0 .. k-1."""
    x = inputs.decode_sweep(131072)
    print(f"[decode parity] sweep every row B={x.B}", flush=True)
    q, w, kc, ks, off = dev(x.q, "bf16"), dev(x.w), dev(x.kc, x.k_dt), dev(x.k_scale), dev(x.kv_off)
    sc = torch.empty(x.n_tok, dtype=torch.float32, device="cuda")
    gi = li.li_index_decode(q, w, kc, ks, off, 131072, x.k, out_scores=sc)
    torch.cuda.synchronize()
    gs = sc.view(x.B, 131072)
    gil = gi.long()
    assert bool((gi >= 0).all()) and bool((gil.diff(dim=1) > 0).all())
    kth = gs.gather(1, gil).min(dim=1).values
    rest = gs.clone()
    rest.scatter_(1, gil, float("-inf"))
    top_rest = rest.max(dim=1).values
    assert bool((kth >= top_rest).all()), "a key above a selected one was left out"
    for b in torch.nonzero(kth == top_rest).flatten().tolist():
        g, sel = gs[b].cpu().numpy(), gi[b].cpu().numpy()
        v = kth[b].item()
        out = np.setdiff1d(np.nonzero(g == v)[0], sel)
        assert out.min() > sel[g[sel] == v].max(), f"row {b}: a tie went to a higher position"
    gi2 = li.li_index_decode(q, w, kc, ks, off, 131072, x.k)
    assert torch.equal(gi, gi2)
    gi3 = li.li_index_decode(q, torch.zeros_like(w), kc, ks, off, 131072, x.k)
    assert torch.equal(gi3.cpu(), torch.arange(x.k, dtype=torch.int32).expand(x.B, x.k))


def check_rows_are_top_k_of_own_scores(gi, gs):
    gil = gi.long()
    assert bool((gi >= 0).all()) and bool((gil.diff(dim=1) > 0).all())
    kth = gs.gather(1, gil).min(dim=1).values
    rest = gs.clone()
    rest.scatter_(1, gil, float("-inf"))
    top_rest = rest.max(dim=1).values
    assert bool((kth >= top_rest).all()), "a key above a selected one was left out"
    for b in torch.nonzero(kth == top_rest).flatten().tolist():
        g, sel = gs[b].cpu().numpy(), gi[b].cpu().numpy()
        out = np.setdiff1d(np.nonzero(g == kth[b].item())[0], sel)
        assert out.min() > sel[g[sel] == kth[b].item()].max(), f"row {b}: a tie went to a higher position"


def test_decode_anchor_shape_k8192_every_row():
    """The HS anchor's shape: B = 16 requests of 131072 fp8 keys with k = 8192
    (4096 keys per scan workgroup, so the scan lists every key and the
    selection resolves the threshold bin from them).  Every row is the top k of
    its own scores; all tied, positions 0 .. k-1."""
    x = inputs.decode_sweep(131072)
    nb, L = 16, 131072
    q, w = dev(x.q[:nb], "bf16"), dev(x.w[:nb])
    kc, ks = dev(x.kc[:nb * L], x.k_dt), dev(x.k_scale[:nb * L])
    off = dev(x.kv_off[:nb + 1])
    k = 8192
    print(f"[decode parity] anchor shape B={nb} L={L} k={k}", flush=True)
    sc = torch.empty(nb * L, dtype=torch.float32, device="cuda")
    gi = li.li_index_decode(q, w, kc, ks, off, L, k, out_scores=sc)
    torch.cuda.synchronize()
    check_rows_are_top_k_of_own_scores(gi, sc.view(nb, L))
    assert torch.equal(gi, li.li_index_decode(q, w, kc, ks, off, L, k))
    gi0 = li.li_index_decode(q, torch.zeros_like(w), kc, ks, off, L, k)
    assert torch.equal(gi0.cpu(), torch.arange(k, dtype=torch.int32).expand(nb, k))


def test_decode_b16_32_lists_every_row():
    """B = 16 requests of 131072 fp8 keys: 32 scan workgroups per request, so
    the selection reads 32 lists, 128 entries of each up front at k <= 2048
    (the rest of a longer list in a second round).  k = 2048 and k = 1500:
    every row is the top k of its own scores, the same without a score
    output, and one request matches the oracle's set; all tied, 0 .. k-1."""
    x = inputs.decode_sweep(131072)
    nb, L = 16, 131072
    q, w = dev(x.q[:nb], "bf16"), dev(x.w[:nb])
    kc, ks = dev(x.kc[:nb * L], x.k_dt), dev(x.k_scale[:nb * L])
    off = dev(x.kv_off[:nb + 1])
    for k in (2048, 1500):
        print(f"[decode parity] B={nb} L={L} k={k} (32 lists)", flush=True)
        sc = torch.empty(nb * L, dtype=torch.float32, device="cuda")
        gi = li.li_index_decode(q, w, kc, ks, off, L, k, out_scores=sc)
        torch.cuda.synchronize()
        check_rows_are_top_k_of_own_scores(gi, sc.view(nb, L))
        assert torch.equal(gi, li.li_index_decode(q, w, kc, ks, off, L, k))
        b = 5
        sl = slice(b * L, (b + 1) * L)
        ri, rs, ra = oracle.index_decode(x.q[b:b + 1], x.q_dt, x.w[b:b + 1], x.kc[sl], x.k_dt, x.k_scale[sl],
                                         np.array([0, L], np.int64), 64, 128, k)
        gs = sc.cpu().numpy()[sl]
        check_scores(gs, rs, ra, what=f"B=16 k={k} b={b}")
        check_sets(gi[b].cpu().numpy(), ri[0], rs, ra, L, what=f"B=16 k={k} b={b}")
    gi0 = li.li_index_decode(q, torch.zeros_like(w), kc, ks, off, L, 2048)
    assert torch.equal(gi0.cpu(), torch.arange(2048, dtype=torch.int32).expand(nb, 2048))
