"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/li.h declares, sizes workspaces, and rejects bad
arguments with the documented status before touching the device."""
import ctypes as C
import os
import re
import subprocess

import pytest

import sparse_attention_token_lightning_amd as li

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "li.h")
FAKE = 0x1000  # never dereferenced: every call below fails host validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(li_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(li.SYMBOLS) == declared_functions()
    # every #define LI_* value the binding mirrors
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (LI_[A-Z0-9_]+)\s+(-?\d+)u?\b", text))
    assert defs, "no LI_ constants parsed"
    for name, value in defs.items():
        if hasattr(li, name):
            assert getattr(li, name) == int(value), name
    for name in ("LI_LATENT_FP16", "LI_LATENT_SPLIT_BF16", "LI_E_VALUE", "LI_MAX_K"):
        assert name in defs and hasattr(li, name), name


def test_library_exports_every_declared_symbol():
    L = li.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", li.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (li_[a-z_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "li.h"\nint main(void){return LI_OK;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-o",
                    str(tmp_path / "t"), str(src)], check=True)


def test_status_strings():
    L = li.lib()
    assert L.li_status_str(li.LI_OK) == b"LI_OK"
    assert L.li_status_str(li.LI_E_WORKSPACE) == b"LI_E_WORKSPACE"
    assert L.li_status_str(li.LI_E_VALUE) == b"LI_E_VALUE"
    assert L.li_status_str(99) == b"LI_E_UNKNOWN"


def test_workspace_queries():
    L = li.lib()
    # rows spanning many scan workgroups (here 256 of 512 keys): the segmented
    # selection, which reads a dense score matrix from the workspace when the
    # caller passes none
    n = 2 * 131072
    with_s = L.li_index_decode_ws(2, n, 131072, 2048, 1)
    without = L.li_index_decode_ws(2, n, 131072, 2048, 0)
    assert without - with_s >= n * 4 and with_s >= 2 * 131072 * 8
    # rows of at most 32 scan workgroups of at least 2k keys (here 16 of 8192):
    # bucket lists (a pair per key) and no dense scores either way
    n = 32 * 131072
    with_s = L.li_index_decode_ws(32, n, 131072, 2048, 1)
    without = L.li_index_decode_ws(32, n, 131072, 2048, 0)
    assert without == with_s and with_s >= 32 * 131072 * 8
    # the same rows with k = 8192 (more than half of a workgroup's keys): segmented
    assert L.li_index_decode_ws(32, n, 131072, 8192, 0) - L.li_index_decode_ws(32, n, 131072, 8192, 1) >= n * 4
    # per-row candidate lists at their worst case: a (key, position) pair per visible key
    assert L.li_index_prefill_ws(4096, 65536, 2048, 0) >= 4096 * 65536 * 8
    # absorbed fp16 queries + scaled weights + scores
    assert L.li_latent_score_group_ws(16, 1 << 21, 131072, 4, 64, 256, 2048, 0) >= 16 * 4 * 64 * 256 * 2 + 4 * (1 << 21) * 4
    assert L.li_hs_refine_ws(16, 8192, 3, 64, 256, 2048, 0) >= 16 * 3 * 8192 * 4
    assert L.li_topk_ws(10, 100, 5) % 256 == 0
    # selection state: candidates of up to max_len / 8192 segments per row
    assert L.li_index_decode_ws(32, 32 * 131072, 131072, 2048, 1) >= 32 * 16 * 8192 * 8


def _decode(**kw):
    a = dict(q=FAKE, q_dt=li.LI_BF16, w=FAKE, k=FAKE, k_dt=li.LI_FP8_E4M3, ks=None, off=FAKE, B=2, n_tok=100,
             max_len=60, H=64, D=128, kk=16, out=FAKE, sc=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    L = li.lib()
    return L.li_index_decode(a["q"], a["q_dt"], a["w"], a["k"], a["k_dt"], a["ks"], a["off"], a["B"], a["n_tok"],
                             a["max_len"], a["H"], a["D"], a["kk"], a["out"], a["sc"], a["ws"], a["wsb"], None)


def test_decode_validation():
    assert _decode(q=None) == li.LI_E_NULL
    assert _decode(off=None) == li.LI_E_NULL
    assert _decode(q_dt=li.LI_FP16) == li.LI_E_DTYPE
    assert _decode(k_dt=li.LI_FP32) == li.LI_E_DTYPE
    assert _decode(kk=0) == li.LI_E_SHAPE
    assert _decode(kk=li.LI_MAX_K + 1) == li.LI_E_UNSUPPORTED
    assert _decode(H=65) == li.LI_E_UNSUPPORTED
    assert _decode(H=0) == li.LI_E_SHAPE
    assert _decode(D=64) == li.LI_E_UNSUPPORTED
    assert _decode(B=-1) == li.LI_E_SHAPE
    assert _decode(wsb=10) == li.LI_E_WORKSPACE
    assert _decode(ws=None) == li.LI_E_NULL
    assert b"workspace" in li.lib().li_last_error()
    assert _decode(B=0) == li.LI_OK  # nothing to do: returns before any launch
    # fp8 keys are addressed with 32-bit byte offsets inside a request
    big = (1 << 25) - 4096
    assert _decode(max_len=big + 1, n_tok=1 << 26) == li.LI_E_UNSUPPORTED
    assert b"max_len" in li.lib().li_last_error()
    assert _decode(max_len=big + 1, n_tok=1 << 26, k_dt=li.LI_BF16, B=0) == li.LI_OK
    assert _decode(max_len=big, n_tok=1 << 26, B=0) == li.LI_OK


def test_noalloc_decode_host_checks():
    """The allocation-free decode rejects a call its static scratch cannot hold,
    and bad arguments, before any device work."""
    L = li.lib()

    def call(B=2, n_tok=100, max_len=60, H=64, sc=None, q=FAKE):
        return L.li_index_decode_noalloc(q, li.LI_BF16, FAKE, FAKE, li.LI_FP8_E4M3, None, FAKE, B, n_tok, max_len,
                                         H, 128, 16, FAKE, sc, None)

    # segmented selection (rows of 4M keys): 128 MiB of dense scores alone
    assert L.li_index_decode_ws(2, 1 << 25, 1 << 22, 16, 0) > li.LI_NOALLOC_SCRATCH_BYTES
    assert call(n_tok=1 << 25, max_len=1 << 22) == li.LI_E_UNSUPPORTED
    assert b"scratch" in L.li_last_error()
    assert call(n_tok=1 << 25, max_len=1 << 22, B=0) == li.LI_E_UNSUPPORTED  # the check does not depend on B
    # bucket lists: a (key, position) pair per key of 64 rows of 128K
    assert L.li_index_decode_ws(64, 64 << 17, 1 << 17, 16, 0) > li.LI_NOALLOC_SCRATCH_BYTES
    assert call(B=64, n_tok=64 << 17, max_len=1 << 17) == li.LI_E_UNSUPPORTED
    assert call(q=None) == li.LI_E_NULL
    assert call(H=65) == li.LI_E_UNSUPPORTED
    assert call(B=-1) == li.LI_E_SHAPE
    assert call(B=0) == li.LI_OK


def test_read_probe_host_checks():
    L = li.lib()
    assert L.li_read_probe(None, 1024, FAKE, None) == li.LI_E_NULL
    assert L.li_read_probe(FAKE, 1024, None, None) == li.LI_E_NULL
    assert L.li_read_probe(FAKE, 1000, FAKE, None) == li.LI_E_SHAPE
    assert L.li_read_probe(FAKE + 8, 1024, FAKE, None) == li.LI_E_SHAPE


def test_mfma_probe_host_checks():
    L = li.lib()
    assert L.li_mfma_probe(li.LI_MFMA_PROBE_F16, 0, 16, None, FAKE, None) == li.LI_E_NULL
    assert L.li_mfma_probe(li.LI_MFMA_PROBE_F16, 0, 16, FAKE, None, None) == li.LI_E_NULL
    assert L.li_mfma_probe(3, 0, 16, FAKE, FAKE, None) == li.LI_E_SHAPE
    assert L.li_mfma_probe(-1, 1, 16, FAKE, FAKE, None) == li.LI_E_SHAPE
    assert L.li_mfma_probe(li.LI_MFMA_PROBE_FP8, 1, 0, FAKE, FAKE, None) == li.LI_E_SHAPE
    assert L.li_mfma_probe(li.LI_MFMA_PROBE_BF16, 0, (1 << 20) + 1, FAKE, FAKE, None) == li.LI_E_SHAPE


def test_prefill_validation():
    L = li.lib()

    def call(**kw):
        a = dict(q=FAKE, q_dt=li.LI_FP8_E4M3, k_dt=li.LI_FP8_E4M3, T=10, Lc=100, qpos0=90, H=64, D=128, kk=5,
                 wsb=1 << 34)
        a.update(kw)
        return L.li_index_prefill(a["q"], a["q_dt"], None, FAKE, FAKE, a["k_dt"], None, a["T"], a["Lc"], a["qpos0"],
                                  a["H"], a["D"], a["kk"], FAKE, None, FAKE, a["wsb"], None)

    assert call(q=None) == li.LI_E_NULL
    assert call(q_dt=li.LI_BF16) == li.LI_E_DTYPE
    assert call(qpos0=91) == li.LI_E_SHAPE
    assert call(qpos0=-1) == li.LI_E_SHAPE
    assert call(D=256) == li.LI_E_UNSUPPORTED
    assert call(wsb=100) == li.LI_E_WORKSPACE
    assert call(T=0, qpos0=0) == li.LI_OK
    # fewer than 8 heads: the fp8 product's error can exceed the score tolerance
    for h in (1, 2, 7):
        assert call(H=h) == li.LI_E_UNSUPPORTED
    assert b"H >= 8" in L.li_last_error()
    assert call(H=8, wsb=100) == li.LI_E_WORKSPACE
    # the cache length is bounded (a wave's candidate rows fit one buffer resource)
    assert call(T=0, Lc=(1 << 26) + 1, qpos0=0) == li.LI_E_SHAPE
    assert b"L <= 67108864" in L.li_last_error()
    assert call(T=0, Lc=1 << 26, qpos0=0) == li.LI_OK


def test_latent_and_hs_validation():
    L = li.lib()

    def lat(**kw):
        a = dict(q_dt=li.LI_BF16, c_dt=li.LI_BF16, cs=None, G=4, H=64, Dc=256, Dh=128, flags=0, kk=8, wsb=1 << 34, B=2)
        a.update(kw)
        return L.li_latent_score_group(FAKE, a["q_dt"], FAKE, FAKE, li.LI_BF16, FAKE, a["c_dt"], a["cs"], FAKE,
                                       a["B"], 1000, 600, a["G"], a["H"], a["Dh"], a["Dc"], a["kk"], FAKE, None,
                                       a["flags"], FAKE, a["wsb"], None)

    assert lat(q_dt=li.LI_FP8_E4M3) == li.LI_E_DTYPE
    assert lat(G=0) == li.LI_E_SHAPE
    assert lat(Dc=160) == li.LI_E_UNSUPPORTED
    assert lat(Dc=192, wsb=1) == li.LI_E_WORKSPACE  # 128 + a 64-value block: accepted
    assert lat(Dh=64) == li.LI_E_UNSUPPORTED
    assert lat(flags=7) == li.LI_E_UNSUPPORTED
    assert lat(flags=2) == li.LI_E_UNSUPPORTED
    # the split form is accepted: the call gets as far as the workspace check
    assert lat(flags=li.LI_LATENT_SPLIT_BF16, wsb=1) == li.LI_E_WORKSPACE
    assert lat(wsb=1) == li.LI_E_WORKSPACE
    assert lat(B=0) == li.LI_OK
    # one head: rejected in both forms; an fp8 latent needs 16 heads; a bf16
    # latent with 2..15 heads is accepted (it runs the split form)
    for fl in (li.LI_LATENT_FP16, li.LI_LATENT_SPLIT_BF16):
        assert lat(H=1, flags=fl) == li.LI_E_UNSUPPORTED
        assert lat(H=2, flags=fl, wsb=1) == li.LI_E_WORKSPACE
    assert lat(H=15, c_dt=li.LI_FP8_E4M3, cs=FAKE) == li.LI_E_UNSUPPORTED
    assert lat(H=16, c_dt=li.LI_FP8_E4M3, cs=FAKE, wsb=1) == li.LI_E_WORKSPACE

    def hs(**kw):
        a = dict(C=8192, Gf=3, H=64, kk=2048, wsb=1 << 34)
        a.update(kw)
        return L.li_hs_refine(FAKE, a["C"], FAKE, li.LI_BF16, FAKE, FAKE, li.LI_BF16, FAKE, li.LI_BF16, None, FAKE,
                              0, a["Gf"], a["H"], 128, 256, a["kk"], FAKE, None, 0, FAKE, a["wsb"], None)

    assert hs(C=0) == li.LI_E_SHAPE
    assert hs(C=70000) == li.LI_E_UNSUPPORTED
    assert hs(Gf=0) == li.LI_E_SHAPE
    assert hs(H=1) == li.LI_E_UNSUPPORTED
    assert hs() == li.LI_OK
    assert L.li_hs_refine(None, 8, FAKE, 0, FAKE, FAKE, 0, FAKE, 0, None, FAKE, 1, 1, 64, 128, 256, 4, FAKE, None,
                          0, FAKE, 1 << 30, None) == li.LI_E_NULL


def test_topk_validation():
    L = li.lib()
    assert L.li_topk(None, 10, None, 1, 10, 1, FAKE, FAKE, 1 << 20, None) == li.LI_E_NULL
    assert L.li_topk(FAKE, 5, None, 1, 10, 1, FAKE, FAKE, 1 << 20, None) == li.LI_E_SHAPE
    assert L.li_topk(FAKE, 10, None, 1, 10, 0, FAKE, FAKE, 1 << 20, None) == li.LI_E_SHAPE
    assert L.li_topk(FAKE, 10, None, 0, 10, 1, FAKE, None, 0, None) == li.LI_OK


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(li, "_lib", None)
    monkeypatch.setattr(li, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        li.lib()


def test_latent_append_validation_and_workspace():
    L = li.lib()

    def ap(**kw):
        a = dict(h=FAKE, h_dt=li.LI_BF16, w=FAKE, w_dt=li.LI_BF16, dst=FAKE, M=4096, d=7168, Dc=256, lat=FAKE,
                 c_dt=li.LI_BF16, sc=None, n_tok=1 << 17, ws=FAKE, wsb=1 << 34)
        a.update(kw)
        return L.li_latent_append(a["h"], a["h_dt"], a["w"], a["w_dt"], a["dst"], a["M"], a["d"], a["Dc"], a["lat"],
                                  a["c_dt"], a["sc"], a["n_tok"], a["ws"], a["wsb"], None)

    assert ap(h=None) == li.LI_E_NULL and ap(dst=None) == li.LI_E_NULL and ap(lat=None) == li.LI_E_NULL
    assert ap(h_dt=li.LI_FP8_E4M3) == li.LI_E_DTYPE and ap(w_dt=li.LI_FP32) == li.LI_E_DTYPE
    assert ap(c_dt=li.LI_FP16) == li.LI_E_DTYPE
    assert ap(c_dt=li.LI_FP8_E4M3) == li.LI_E_NULL  # fp8 output needs its block scales
    assert ap(M=-1) == li.LI_E_SHAPE and ap(d=0) == li.LI_E_SHAPE and ap(n_tok=0) == li.LI_E_SHAPE
    assert ap(d=7168 + 32) == li.LI_E_UNSUPPORTED
    assert ap(Dc=160) == li.LI_E_UNSUPPORTED
    assert ap(Dc=192, wsb=1) == li.LI_E_WORKSPACE  # accepted: stops at the workspace check, before any launch
    assert ap(wsb=1) == li.LI_E_WORKSPACE
    assert ap(M=0, ws=None, wsb=0) == li.LI_OK
    assert ap(M=0, h=None, dst=None, ws=None, wsb=0) == li.LI_OK
    assert ap(w=None) == li.LI_E_NULL
    # partial sums of the K split: [S][M][Dc] fp32, S > 1 for a 4096-token chunk
    need = L.li_latent_append_ws(4096, 7168, 256, li.LI_BF16)
    assert need >= 2 * 4096 * 256 * 4 and need % (4096 * 256 * 4) == 0
    assert L.li_latent_append_ws(0, 7168, 256, li.LI_BF16) == 0
    # one K step covers d_model = 64: bf16 output is written directly, fp8 output goes through the split sum
    assert L.li_latent_append_ws(16, 64, 128, li.LI_BF16) == 0
    assert L.li_latent_append_ws(16, 64, 128, li.LI_FP8_E4M3) >= 16 * 128 * 4


def test_indexcache_plan():
    # uniform retention over DeepSeek-V3.2's 61 indexer layers: 61, 31 and 16 scans per token
    for r, full in ((1, 61), (2, 31), (4, 16)):
        n, src = li.li_indexcache_plan(61, r)
        assert n == full
        assert all(src[l] == l - l % r for l in range(61))
    # the page's worked group F S S S F: layers 13-15 attend layer 12's selection
    roles = [0] * 20
    roles[0] = roles[12] = roles[16] = 1
    n, src = li.li_indexcache_plan(20, roles=roles)
    assert n == 3 and src[12:17] == [12, 12, 12, 12, 16] and src[:12] == [0] * 12 and src[19] == 16
    # every layer F is native DSA
    assert li.li_indexcache_plan(5, roles=[1] * 5) == (5, [0, 1, 2, 3, 4])
    L = li.lib()
    assert L.li_indexcache_plan(None, 4, 1, None) == -li.LI_E_NULL
    with pytest.raises(li.LiError):
        li.li_indexcache_plan(0, 1)
    with pytest.raises(li.LiError):
        li.li_indexcache_plan(8, 0)
    with pytest.raises(li.LiError):
        li.li_indexcache_plan(3, roles=[0, 1, 1])


def test_latentindex_storage_closed_form():
    """LatentIndex page, Abstract: -61.1% logical indexer-cache storage at G = 4
    on DeepSeek-V3.2.  With 61 indexed layers (Table 5), layer 0 independent,
    15 groups of 4, native fp8 keys of 64 + 64 dims with one fp32 scale, and a
    shared fp8 latent of 64 + 128 dims with one fp32 scale per started
    128-value block, the saving is 1 - (132 + 15 * 200) / (61 * 132)."""
    L = li.lib()
    key = L.li_key_row_bytes(128, li.LI_FP8_E4M3)
    lat = L.li_latent_row_bytes(64 + 128, li.LI_FP8_E4M3)
    assert (key, lat) == (132, 200)
    saving = 1 - (key + 15 * lat) / (61 * key)
    assert round(saving * 100, 1) == 61.1
    # and it is a layout the library takes: an fp8 latent of 192 values per row
    # passes the host checks of the group scan (this call stops at the workspace check)
    assert L.li_latent_score_group(FAKE, li.LI_BF16, FAKE, FAKE, li.LI_BF16, FAKE, li.LI_FP8_E4M3, FAKE, FAKE, 2, 1000,
                                   600, 4, 64, 128, 64 + 128, 8, FAKE, None, 0, FAKE, 1, None) == li.LI_E_WORKSPACE
    assert L.li_latent_row_bytes(256, li.LI_FP8_E4M3) == 264 and L.li_latent_row_bytes(256, li.LI_BF16) == 512
    assert L.li_key_row_bytes(128, li.LI_BF16) == 256 and L.li_key_row_bytes(0, li.LI_BF16) == 0
    assert L.li_latent_row_bytes(128, li.LI_FP32) == 0
