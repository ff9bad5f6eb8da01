"""The entry points under HIP graph capture: each call is captured once into a
torch.cuda.CUDAGraph (caller-provided workspace and outputs, so nothing is
allocated inside the capture), then replayed several times with eager work
and synchronisations between the replays; every replay must reproduce the
eager call's indices (and scores) bit for bit."""
import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def check_replays(run, outs, what):
    """run() enqueues the call on the current stream, writing into `outs`."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outs:  # eager work between replays: clobber the outputs
            o.fill_(-7)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.int32), r.view(torch.int32)), f"{what}: replay {rep} differs"
        print(f"[graph] {what}: replay {rep} ok ({float(junk):.1f})", flush=True)


def test_decode_graph():
    x = inputs.make_decode(901, [5000, 3000, 0, 777, 20000], k=512)
    q, w, kc, ks, off = dev(x.q, "bf16"), dev(x.w), dev(x.kc, "fp8_e4m3"), dev(x.k_scale), dev(x.kv_off)
    L = int(x.lens.max())
    out = torch.empty((x.B, x.k), dtype=torch.int32, device="cuda")
    sc = torch.empty(x.n_tok, dtype=torch.float32, device="cuda")
    ws = torch.empty(li.lib().li_index_decode_ws(x.B, x.n_tok, L, x.k, 1), dtype=torch.uint8, device="cuda")
    check_replays(lambda: li.li_index_decode(q, w, kc, ks, off, L, x.k, out_idx=out, out_scores=sc, ws=ws),
                  [out, sc], "decode")


def test_prefill_graph():
    x = inputs.make_prefill(902, 48, 5000, k=256)
    q, qs, w, kc, ks = dev(x.q, "fp8_e4m3"), dev(x.q_scale), dev(x.w), dev(x.kc, "fp8_e4m3"), dev(x.k_scale)
    out = torch.empty((x.T, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(li.lib().li_index_prefill_ws(x.T, x.L, x.k, 0), dtype=torch.uint8, device="cuda")
    check_replays(lambda: li.li_index_prefill(q, qs, w, kc, ks, x.qpos0, x.k, out_idx=out, ws=ws), [out],
                  "prefill")


@pytest.mark.parametrize("flags", [li.LI_LATENT_FP16, li.LI_LATENT_SPLIT_BF16])
def test_latent_graph(flags):
    x = inputs.make_latent(903, [3000, 1200, 0], G=4, k=256)
    q, w, wd, lat, off = dev(x.q, "bf16"), dev(x.w), dev(x.w_dec, "bf16"), dev(x.latent, "bf16"), dev(x.kv_off)
    L = int(np.diff(x.kv_off).max())
    out = torch.empty((x.B, x.G, x.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(li.lib().li_latent_score_group_ws(x.B, x.n_tok, L, x.G, x.H, x.Dc, x.k, 0),
                     dtype=torch.uint8, device="cuda")
    check_replays(lambda: li.li_latent_score_group(q, w, wd, lat, None, off, L, x.k, out_idx=out, flags=flags,
                                                   ws=ws), [out], f"latent flags={flags}")


def test_hs_graph():
    h = inputs.make_hs(904, [9000, 3000, 500], C=2048, Gf=3, k=512)
    a, f = h.anchor, h.followers
    aq, aw, akc, aks, off = dev(a.q, "bf16"), dev(a.w), dev(a.kc, a.k_dt), dev(a.k_scale), dev(a.kv_off)
    fq, fw, fwd, lat = dev(f.q, "bf16"), dev(f.w), dev(f.w_dec, "bf16"), dev(f.latent, "bf16")
    La = int(np.diff(a.kv_off).max())
    cand = torch.empty((a.B, h.C), dtype=torch.int32, device="cuda")
    fout = torch.empty((a.B, f.G, f.k), dtype=torch.int32, device="cuda")
    ws_a = torch.empty(li.lib().li_index_decode_ws(a.B, a.n_tok, La, h.C, 0), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(li.lib().li_hs_refine_ws(a.B, h.C, f.G, f.H, f.Dc, f.k, 0), dtype=torch.uint8, device="cuda")

    def run():
        li.li_index_decode(aq, aw, akc, aks, off, La, h.C, out_idx=cand, ws=ws_a)
        li.li_hs_refine(cand, fq, fw, fwd, lat, None, off, f.k, out_idx=fout, ws=ws_f)

    check_replays(run, [cand, fout], "hs")


def test_append_graph():
    # no old tokens: every cache row is appended to, so each replay rewrites the whole output
    x = inputs.make_append(905, [0, 0, 0], [300, 5, 77], d_model=2048)
    assert x.n_tok == x.M
    h, wenc, dst = dev(x.h, "bf16"), dev(x.w_enc, "bf16"), dev(x.dst_row)
    lat = torch.zeros((x.n_tok, x.Dc), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(li.lib().li_latent_append_ws(x.M, x.d_model, x.Dc, li.LI_BF16), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0  # the split path (partial sums + reduction) is the one captured
    check_replays(lambda: li.li_latent_append(h, wenc, dst, lat, ws=ws), [lat], "append")


def test_two_stream_mli_graph():
    """Lagged selection (Multi-layer Indexer): layer l attends layer l-1's
    selection on the capturing stream while its own indexer runs on a second
    stream; the captured graph's replays match the eager run bit for bit."""
    from sparse_attention_token_lightning_amd.inputs import make_attention, make_decode
    n_layers, k = 3, 256
    dec = [make_decode(910 + l, [3000, 1500], k=k) for l in range(n_layers)]
    att = [make_attention(920 + l, [3000, 1500], H=64, k=k) for l in range(n_layers)]
    d_in = [(dev(x.q, "bf16"), dev(x.w), dev(x.kc, "fp8_e4m3"), dev(x.k_scale), dev(x.kv_off)) for x in dec]
    a_in = [(dev(x.q, "bf16"), dev(x.kv, "bf16")) for x in att]
    L = 3000
    sel = [torch.empty((2, k), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    outs = [torch.empty((2, 64, 512), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ws_i = torch.empty(li.lib().li_index_decode_ws(2, dec[0].n_tok, L, k, 0), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(li.lib().li_sparse_attention_ws(2, 64, k), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()

    def indexer(l):
        q, w, kc, ks, off = d_in[l]
        li.li_index_decode(q, w, kc, ks, off, L, k, out_idx=sel[l], ws=ws_i)

    def attention(l, s):
        q, kv = a_in[l]
        li.li_sparse_attention(q, kv, sel[s], d_in[l][4], att[l].scale, out=outs[l], ws=ws_a)

    def run():
        cur = torch.cuda.current_stream()
        indexer(0)
        attention(0, 0)
        for l in range(1, n_layers):
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                indexer(l)
            attention(l, l - 1)
            cur.wait_stream(side)

    check_replays(run, sel + outs, "mli two-stream")
