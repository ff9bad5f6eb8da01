"""li_index_decode_noalloc: the decode with the library's static device
scratch as its workspace, for callers that cannot allocate.  Its results must
equal li_index_decode's bit for bit (same kernels), on consecutive calls of
different sizes that share the one scratch array, and a call too large for the
scratch is rejected before any device work."""
import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as li
from sparse_attention_token_lightning_amd import inputs
from _parity import dev

pytestmark = pytest.mark.gpu


def both(x, with_scores):
    q, w, kc, ks, off = dev(x.q, "bf16"), dev(x.w), dev(x.kc, x.k_dt), dev(x.k_scale), dev(x.kv_off)
    max_len = int(x.lens.max(initial=0))
    s_ref = torch.full((max(x.n_tok, 1),), float("nan"), device="cuda") if with_scores else None
    s_na = torch.full((max(x.n_tok, 1),), float("nan"), device="cuda") if with_scores else None
    ref = li.li_index_decode(q, w, kc, ks, off, max_len, x.k, out_scores=s_ref)
    got = torch.full((x.B, x.k), -7, dtype=torch.int32, device="cuda")
    li.li_index_decode_noalloc(q, w, kc, ks, off, max_len, x.k, got, out_scores=s_na)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    if with_scores:
        assert torch.equal(s_na.view(torch.int32), s_ref.view(torch.int32))
    return got


def test_noalloc_decode_matches_the_workspace_decode_on_consecutive_calls():
    # 1: the full B = 32 x 131072 fp8 decode (about 50 MiB of scratch: scores,
    #    histograms and candidates all in the static array)
    x = inputs.decode_sweep(131072)
    need = li.lib().li_index_decode_ws(x.B, x.n_tok, 131072, x.k, 0)
    print(f"[noalloc] B={x.B} L=131072 scratch {need / 2**20:.1f} MiB", flush=True)
    assert need <= li.LI_NOALLOC_SCRATCH_BYTES
    both(x, with_scores=False)
    del x
    # 2: a smaller ragged batch right after, with a score output, so what the
    #    first call left in the scratch must not leak into it
    x = inputs.make_decode(1201, [30000, 9000, 40, 0, 17000], k=2048)
    print(f"[noalloc] ragged B={x.B} n_tok={x.n_tok}", flush=True)
    both(x, with_scores=True)
    # 3: and a smaller one again, rows shorter than k, bf16 keys
    x = inputs.make_decode(1202, [700, 1500], k=1024, k_dt="bf16")
    print(f"[noalloc] bf16 B={x.B} n_tok={x.n_tok}", flush=True)
    both(x, with_scores=False)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    x = inputs.make_decode(1203, [64], k=16)
    q, w, kc, ks, off = dev(x.q, "bf16"), dev(x.w), dev(x.kc, x.k_dt), dev(x.k_scale), dev(x.kv_off)
    out = torch.empty((1, 16), dtype=torch.int32, device="cuda")
    # n_tok and max_len as the caller states them size the scratch: rows of up
    # to 4M keys select through a dense score buffer, 128 MiB for 2^25 keys
    with pytest.raises(li.LiError) as e:
        li.lib()
        st = li.lib().li_index_decode_noalloc(li._ptr(q), li.LI_BF16, li._ptr(w), li._ptr(kc), li.LI_FP8_E4M3,
                                              li._ptr(ks), li._ptr(off), 1, 1 << 25, 1 << 22, 64, 128, 16,
                                              li._ptr(out), None, None)
        li._check(st)
    assert e.value.status == li.LI_E_UNSUPPORTED and "scratch" in str(e.value)
