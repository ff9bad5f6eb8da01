"""GPU parity of li_latent_append (the LatentIndex shared-latent append)
against the CPU oracle.

Integer-valued inputs make every fp32 partial sum exact, so there the stored
bf16 codes must equal the oracle's bit for bit.  With normal inputs the
kernel's fp32 sum y may differ from the exact sum e by up to the summation
bound b = (d_model + 64) * 2^-24 * sum_i |h_i w_i|; rounding is monotone, so a
stored code that differs from the oracle's must lie between the roundings of
e - b and e + b (near cancellation that can be several bf16 steps of a tiny
result), and such codes must stay rare."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import dev

pytestmark = pytest.mark.gpu

SENTINEL = -7.0  # initial value of every latent row; rows not appended to must keep it

def bf16_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16).double().numpy()

def run_append(x, ws=None):
    lat = torch.full((x.n_tok, x.Dc), SENTINEL, dtype=torch.bfloat16, device="cuda")
    li.li_latent_append(dev(x.h, "bf16"), dev(x.w_enc, "bf16"), dev(x.dst_row), lat, ws=ws)
    torch.cuda.synchronize()
    return lat

def rows_of(lat, rows):
    r = torch.from_numpy(np.asarray(rows, np.int64)).cuda()
    return lat.index_select(0, r).view(torch.int16).cpu().numpy().view(np.uint16)

def untouched_keep_sentinel(lat, dst, what):
    changed = (lat != SENTINEL).any(dim=1).nonzero().flatten().cpu().numpy()
    assert np.isin(changed, dst).all(), f"{what}: rows outside dst_row were written: {changed[~np.isin(changed, dst)][:8]}"

def check_codes(got, ref, exact, h_rows, w_enc, d_model, what, exact_only=False):
    """got/ref [m][Dc] bf16 codes, exact [m][Dc] fp64 sums of the same rows."""
    diff = got != ref
    nd = int(diff.sum())
    print(f"[append parity] {what}: {nd} of {got.size} codes differ from the oracle", flush=True)
    if exact_only:
        assert nd == 0, f"{what}: integer-valued sums must round identically"
        return
    if nd == 0:
        return
    hv = np.abs(bf16_values(h_rows))
    wv = np.abs(bf16_values(w_enc))
    bound = ((d_model + 64) * 2.0 ** -24 * (hv @ wv.T))[diff]
    e = exact[diff]
    lo = bf16_values(np.array([oracle.encode_bf16(v) for v in e - bound], np.uint16))
    hi = bf16_values(np.array([oracle.encode_bf16(v) for v in e + bound], np.uint16))
    gv = bf16_values(got[diff])
    assert np.all((lo <= gv) & (gv <= hi)), f"{what}: a differing code is not explained by fp32 summation"
    assert nd <= max(4, got.size // 200), f"{what}: too many boundary cases ({nd})"

def append_parity(x, what, rows=None, exact_only=False):
    """Compare the rows `rows` (indices into the M new tokens; all by default)."""
    print(f"[append parity] {what} M={x.M} d_model={x.d_model} Dc={x.Dc} n_tok={x.n_tok}", flush=True)
    lat = run_append(x)
    untouched_keep_sentinel(lat, x.dst_row, what)
    m = np.arange(x.M) if rows is None else np.asarray(rows)
    got = rows_of(lat, x.dst_row[m])
    sub_dst = np.arange(m.size, dtype=np.int64)
    ref, exact = oracle.latent_append(x.h[m], "bf16", x.w_enc, "bf16", sub_dst, np.zeros((m.size, x.Dc), np.uint16))
    check_codes(got, ref, exact, x.h[m], x.w_enc, x.d_model, what, exact_only)
    return lat

def test_append_integer_exact_ragged_requests():
    x = inputs.make_append(401, [5, 0, 300, 17], [130, 1, 200, 3], d_model=1024, dist="int")
    append_parity(x, "int ragged d1024", exact_only=True)

def test_append_integer_exact_full_hidden_size():
    x = inputs.make_append(402, [1000], [200], d_model=7168, dist="int")
    append_parity(x, "int d7168", exact_only=True)

def test_append_normal_ragged_dc256_and_dc128():
    append_parity(inputs.make_append(403, [10, 4000, 0], [150, 7, 143], d_model=2048), "normal Dc256 d2048")
    append_parity(inputs.make_append(404, [64, 3], [129, 255], d_model=1536, Dc=128), "normal Dc128 d1536")

def test_append_one_split_writes_the_cache_directly():
    # d_model = 64 is one K step, hence one split: no partial sums, no workspace;
    # d_model = 128 splits its two K steps
    for d, seed in ((64, 405), (128, 406)):
        assert (li.lib().li_latent_append_ws(300, d, 256, li.LI_BF16) == 0) == (d == 64)
        append_parity(inputs.make_append(seed, [2, 9], [131, 126], d_model=d, dist="int"), f"int d{d}",
                      exact_only=True)
        append_parity(inputs.make_append(seed + 10, [2, 9], [131, 126], d_model=d, Dc=128), f"normal d{d} Dc128")

def test_append_single_token_and_empty_batch():
    append_parity(inputs.make_append(407, [77], [1], d_model=7168), "M=1 d7168")
    x = inputs.make_append(408, [5, 6], [0, 0], d_model=256)
    assert x.M == 0
    lat = run_append(x)
    assert bool((lat == SENTINEL).all())

def test_append_prefill_chunk_full_size_sampled_rows():
    x = inputs.append_prefill()
    rng = np.random.default_rng(409)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(x.M - 8, x.M), np.arange(120, 136),
                                     rng.choice(x.M, 40, replace=False)]))
    lat = append_parity(x, x.name, rows=rows)
    # every appended row is finite
    new = lat[torch.from_numpy(x.dst_row).cuda()].float()
    assert bool(torch.isfinite(new).all())

def test_append_decode_step_full_size():
    x = inputs.append_decode()
    append_parity(x, x.name)

def test_append_ignores_workspace_contents_and_repeats():
    x = inputs.make_append(410, [40, 7], [300, 90], d_model=3072)
    need = li.lib().li_latent_append_ws(x.M, x.d_model, x.Dc, li.LI_BF16)
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    first = run_append(x, ws=ws)
    again = run_append(x, ws=ws)
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    small = inputs.make_append(411, [3], [50], d_model=3072)
    append_parity(small, "after a larger call")
    ws.fill_(255)
    third = run_append(x, ws=ws)
    assert torch.equal(first.view(torch.int16), third.view(torch.int16))

def test_append_debug_validation_rejects_rows_outside_the_cache(monkeypatch):
    x = inputs.make_append(412, [10], [20], d_model=256)
    x.dst_row = x.dst_row.copy()
    x.dst_row[7] = x.n_tok  # one past the cache
    monkeypatch.setenv("LI_DEBUG_VALIDATE", "1")
    lat = torch.full((x.n_tok, x.Dc), SENTINEL, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(li.LiError) as e:
        li.li_latent_append(dev(x.h, "bf16"), dev(x.w_enc, "bf16"), dev(x.dst_row), lat)
    assert e.value.status == li.LI_E_VALUE and "dst_row" in str(e.value)
    torch.cuda.synchronize()
    assert bool((lat == SENTINEL).all())


def fp8_append_parity(x, what, exact_only=False):
    """fp8 output: codes and block scales against the oracle's fp32 quantisation.
    Integer inputs: identical.  Normal inputs: the kernel's fp32 sum y lies within
    b of the exact sum e, so its block max within b_max of the exact one, its
    scale within that / 448 (plus fp32 rounding), and each code between the
    E4M3 roundings of (e - b) / scale and (e + b) / scale."""
    print(f"[append parity] {what} fp8 M={x.M} d_model={x.d_model} Dc={x.Dc}", flush=True)
    nb = (x.Dc + 127) // 128  # 128-value blocks from the row's start (Dc = 192: 128 + 64)
    blk = np.arange(x.Dc) // 128
    lat = torch.zeros((x.n_tok, x.Dc), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sc = torch.zeros((x.n_tok, nb), dtype=torch.float32, device="cuda")
    li.li_latent_append(dev(x.h, "bf16"), dev(x.w_enc, "bf16"), dev(x.dst_row), lat, c_scale=sc)
    torch.cuda.synchronize()
    rows = torch.from_numpy(x.dst_row).cuda()
    got = lat.view(torch.uint8).index_select(0, rows).cpu().numpy()
    gsc = sc.index_select(0, rows).cpu().numpy()
    ref, rsc, exact = oracle.latent_append(x.h, "bf16", x.w_enc, "bf16", np.arange(x.M), np.zeros((x.M, x.Dc), np.uint8),
                                           c_scale=np.zeros((x.M, nb), np.float32))
    nd = int((got != ref).sum())
    print(f"[append parity] {what} fp8: {nd} of {got.size} codes and {int((gsc != rsc).sum())} scales differ", flush=True)
    if exact_only:
        assert np.array_equal(got, ref) and np.array_equal(gsc, rsc)
        return
    hv = np.abs(bf16_values(x.h))
    wv = np.abs(bf16_values(x.w_enc))
    b = (x.d_model + 64) * 2.0 ** -24 * (hv @ wv.T)
    amax = np.stack([np.abs(exact[:, blk == j]).max(axis=1) for j in range(nb)], 1)
    bmax = np.stack([b[:, blk == j].max(axis=1) for j in range(nb)], 1)
    assert np.all(np.abs(gsc.astype(np.float64) * 448 - amax) <= bmax + 2.0 ** -22 * amax), f"{what}: scales"
    s = gsc.astype(np.float64)[:, blk]
    dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    diff = got != ref
    if diff.any():
        e, bb, ss = exact[diff], b[diff], s[diff]
        lo = dec(np.array([oracle.encode_e4m3(v) for v in (e - bb) / ss], np.uint8))
        hi = dec(np.array([oracle.encode_e4m3(v) for v in (e + bb) / ss], np.uint8))
        g = dec(got[diff])
        assert np.all((lo <= g) & (g <= hi)), f"{what}: a code not explained by fp32 summation"
    assert nd <= max(4, got.size // 100), f"{what}: too many boundary codes ({nd})"
    untouched = np.setdiff1d(np.arange(x.n_tok), x.dst_row)
    if untouched.size:
        u = torch.from_numpy(untouched[:4096]).cuda()
        assert int(lat.view(torch.uint8).index_select(0, u).count_nonzero()) == 0


def test_append_fp8_integer_exact():
    fp8_append_parity(inputs.make_append(413, [5, 0, 300], [130, 1, 70], d_model=1024, dist="int"), "int d1024",
                      exact_only=True)
    fp8_append_parity(inputs.make_append(414, [9], [40], d_model=64, Dc=128, dist="int"), "int d64 Dc128",
                      exact_only=True)


def test_append_fp8_normal_and_prefill_chunk():
    fp8_append_parity(inputs.make_append(415, [10, 4000], [150, 77], d_model=2048), "normal d2048")
    fp8_append_parity(inputs.make_append(416, [64, 3], [129, 255], d_model=1536, Dc=128), "normal Dc128")


def test_appended_fp8_latent_feeds_the_scan():
    # The fp8 rows the append writes are what the latent scan reads.  With
    # integer-valued inputs the appended codes and scales equal the oracle's,
    # so the GPU scan of the GPU-appended cache is checked against the oracle's
    # scan of the oracle-appended cache.
    x = inputs.make_append(417, [0, 0], [700, 300], d_model=512, dist="int")
    lat = torch.zeros((x.n_tok, x.Dc), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    sc = torch.zeros((x.n_tok, 2), dtype=torch.float32, device="cuda")
    li.li_latent_append(dev(x.h, "bf16"), dev(x.w_enc, "bf16"), dev(x.dst_row), lat, c_scale=sc)
    codes, scales, _ = oracle.latent_append(x.h, "bf16", x.w_enc, "bf16", x.dst_row, np.zeros((x.n_tok, x.Dc), np.uint8),
                                            c_scale=np.zeros((x.n_tok, 2), np.float32))
    torch.cuda.synchronize()
    assert np.array_equal(lat.view(torch.uint8).cpu().numpy(), codes) and np.array_equal(sc.cpu().numpy(), scales)
    y = inputs.make_latent(418, [700, 300], G=2, k=64)
    ls = torch.empty((2, x.n_tok), dtype=torch.float32, device="cuda")
    li.li_latent_score_group(dev(y.q, "bf16"), dev(y.w), dev(y.w_dec, "bf16"), lat, sc, dev(y.kv_off), 700, y.k,
                             out_scores=ls)
    torch.cuda.synchronize()
    _, rs, ra = oracle.latent_score_group(y.q, "bf16", y.w, y.w_dec, "bf16", codes, "fp8_e4m3", scales, y.kv_off,
                                          2, y.H, 128, 256, y.k, c_blocks=2)
    err = np.abs(ls.cpu().numpy().astype(np.float64) - rs)
    assert np.all(err <= 2e-3 * ra)


def test_append_dc192_bf16_and_fp8():
    """Dc = 192 (the shared latent of 64 rotary + 128 other dims): the
    contraction's column tiles do not split evenly over its threads, and the
    fp8 output has a 128-value block and a 64-value tail block."""
    x = inputs.make_append(419, [5, 0, 300], [130, 1, 70], d_model=1024, Dc=192, dist="int")
    append_parity(x, "int d1024 Dc192", exact_only=True)
    fp8_append_parity(x, "int d1024 Dc192", exact_only=True)
    x = inputs.make_append(420, [10, 4000], [150, 77], d_model=2048, Dc=192)
    append_parity(x, "normal d2048 Dc192")
    fp8_append_parity(x, "normal d2048 Dc192")
    x = inputs.make_append(421, [3], [40], d_model=64, Dc=192)
    append_parity(x, "normal d64 Dc192 (one split, direct write)")
