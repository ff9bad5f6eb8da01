"""Python binding of the MI355X lightning-indexer library (libli.so).

Argument marshalling only: every step of the scan, the selection, the latent
absorption and the HS rescoring runs in the HIP kernels behind the C ABI
declared in ``include/li.h``.  The functions carry the ABI's names and take
torch tensors that already live on the GPU; torch supplies device memory (the
workspace and default outputs) and the current stream.

There is no fallback: if ``libli.so`` has not been built, or the GPU is
missing, every call raises.
"""
import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libli.so")

LI_OK, LI_E_NULL, LI_E_SHAPE, LI_E_DTYPE, LI_E_WORKSPACE, LI_E_UNSUPPORTED, LI_E_HIP, LI_E_VALUE = range(8)
LI_BF16, LI_FP8_E4M3, LI_FP16, LI_FP32 = range(4)
LI_LATENT_FP16 = 0
LI_LATENT_SPLIT_BF16 = 1
LI_MAX_K = 16384
LI_NOALLOC_SCRATCH_BYTES = 64 << 20
LI_READ_PROBE_SINK_WORDS = 8192
LI_MFMA_PROBE_F16, LI_MFMA_PROBE_BF16, LI_MFMA_PROBE_FP8 = 0, 1, 2
LI_MFMA_PROBE_WAVES = 8192
LI_MFMA_PROBE_PRODUCTS_PER_ITER = 16
LI_MFMA_PROBE_SINK_WORDS = 8192
LI_MFMA_PROBE_CLOCK_WORDS = 4096

# Every symbol include/li.h declares.
SYMBOLS = ("li_index_decode", "li_index_decode_ws", "li_index_decode_noalloc", "li_index_prefill", "li_index_prefill_ws",
           "li_latent_score_group", "li_latent_score_group_ws", "li_hs_refine", "li_hs_refine_ws",
           "li_latent_append", "li_latent_append_ws", "li_sparse_attention", "li_sparse_attention_ws", "li_key_row_bytes", "li_latent_row_bytes", "li_indexcache_plan", "li_topk", "li_topk_ws", "li_status_str", "li_last_error", "li_trace_events", "li_trace_count", "li_read_probe", "li_mfma_probe")

_lib = None


class LiError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{detail}")


def lib():
    """Load libli.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run sparse_attention_token_lightning_amd/build.py")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_uint32
        L.li_index_decode.argtypes = [vp, i32, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.li_index_decode_ws.argtypes = [i32, i64, i32, i32, i32]
        L.li_index_decode_noalloc.argtypes = [vp, i32, vp, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp]
        L.li_index_prefill.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.li_index_prefill_ws.argtypes = [i32, i32, i32, i32]
        L.li_latent_score_group.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                            i32, vp, vp, u32, vp, sz, vp]
        L.li_latent_score_group_ws.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32]
        L.li_hs_refine.argtypes = [vp, i32, vp, i32, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                   vp, u32, vp, sz, vp]
        L.li_hs_refine_ws.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.li_latent_append.argtypes = [vp, i32, vp, i32, vp, i32, i32, i32, vp, i32, vp, i64, vp, sz, vp]
        L.li_latent_append_ws.argtypes = [i32, i32, i32, i32]
        L.li_sparse_attention.argtypes = [vp, i32, vp, i32, vp, vp, i32, i64, i32, i32, i32, i32, C.c_float, vp, vp, sz,
                                          vp]
        L.li_sparse_attention_ws.argtypes = [i32, i32, i32]
        for f in ("li_key_row_bytes", "li_latent_row_bytes"):
            getattr(L, f).restype = sz
            getattr(L, f).argtypes = [i32, i32]
        L.li_indexcache_plan.restype = i32
        L.li_indexcache_plan.argtypes = [vp, i32, i32, vp]
        L.li_topk.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, sz, vp]
        L.li_topk_ws.argtypes = [i32, i32, i32]
        for f in ("li_index_decode", "li_index_decode_noalloc", "li_index_prefill", "li_latent_score_group", "li_hs_refine",
                  "li_latent_append",
                  "li_sparse_attention", "li_topk"):
            getattr(L, f).restype = C.c_int32
        for f in ("li_index_decode_ws", "li_index_prefill_ws", "li_latent_score_group_ws", "li_hs_refine_ws",
                  "li_latent_append_ws", "li_sparse_attention_ws", "li_topk_ws"):
            getattr(L, f).restype = C.c_size_t
        L.li_status_str.argtypes = [i32]
        L.li_status_str.restype = C.c_char_p
        L.li_last_error.argtypes = []
        L.li_last_error.restype = C.c_char_p
        L.li_trace_events.argtypes = [vp, i32]
        L.li_trace_events.restype = None
        L.li_trace_count.argtypes = []
        L.li_trace_count.restype = i32
        L.li_read_probe.argtypes = [vp, sz, vp, vp]
        L.li_read_probe.restype = i32
        L.li_mfma_probe.argtypes = [i32, i32, i32, vp, vp, vp]
        L.li_mfma_probe.restype = i32
        _lib = L
    return _lib


def _check(st):
    if st != LI_OK:
        L = lib()
        raise LiError(st, f"{L.li_status_str(st).decode()}: {L.li_last_error().decode()}")


_DT = {torch.bfloat16: LI_BF16, torch.float8_e4m3fn: LI_FP8_E4M3, torch.float16: LI_FP16, torch.float32: LI_FP32}


def _dt(t):
    if t.dtype not in _DT:
        raise TypeError(f"unsupported element type {t.dtype}")
    return _DT[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def li_index_decode(q, w, k_cache, k_scale, kv_off, max_len, k, out_idx=None, out_scores=None, ws=None,
                    stream=None):
    """Decode scan + top-k.  q [B,H,D] bf16, w [B,H] fp32, k_cache [n_tok,D] bf16 or
    float8_e4m3fn, k_scale [n_tok] fp32 or None, kv_off [B+1] int64.  Returns
    out_idx [B,k] int32."""
    B, H, D = q.shape
    n_tok = k_cache.shape[0]
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
    L = lib()
    need = L.li_index_decode_ws(B, n_tok, max_len, k, int(out_scores is not None))
    wst, wsb = _workspace(need, q.device, ws)
    _check(L.li_index_decode(_ptr(q), _dt(q), _ptr(w), _ptr(k_cache), _dt(k_cache), _ptr(k_scale), _ptr(kv_off), B,
                             n_tok, max_len, H, D, k, _ptr(out_idx), _ptr(out_scores), _ptr(wst), wsb,
                             _stream(stream)))
    return out_idx


def li_index_decode_noalloc(q, w, k_cache, k_scale, kv_off, max_len, k, out_idx, out_scores=None, stream=None):
    """li_index_decode with the library's static device scratch as workspace
    (nothing is allocated, here or in the library): the caller passes out_idx
    [B,k] int32 (and out_scores [n_tok] fp32 or None)."""
    B, H, D = q.shape
    n_tok = k_cache.shape[0]
    _check(lib().li_index_decode_noalloc(_ptr(q), _dt(q), _ptr(w), _ptr(k_cache), _dt(k_cache), _ptr(k_scale),
                                         _ptr(kv_off), B, n_tok, max_len, H, D, k, _ptr(out_idx), _ptr(out_scores),
                                         _stream(stream)))
    return out_idx


def li_index_prefill(q, q_scale, w, k_cache, k_scale, qpos0, k, out_idx=None, out_scores=None, ws=None,
                     stream=None):
    """Causal prefill scan + top-k.  q [T,H,D] float8_e4m3fn, q_scale [T] or None,
    w [T,H] fp32, k_cache [L,D] float8_e4m3fn, k_scale [L] or None.  Returns
    out_idx [T,k] int32."""
    T, H, D = q.shape
    Lc = k_cache.shape[0]
    if out_idx is None:
        out_idx = torch.empty((T, k), dtype=torch.int32, device=q.device)
    L = lib()
    need = L.li_index_prefill_ws(T, Lc, k, int(out_scores is not None))
    wst, wsb = _workspace(need, q.device, ws)
    _check(L.li_index_prefill(_ptr(q), _dt(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _dt(k_cache), _ptr(k_scale),
                              T, Lc, qpos0, H, D, k, _ptr(out_idx), _ptr(out_scores), _ptr(wst), wsb,
                              _stream(stream)))
    return out_idx


def li_latent_score_group(q, w, w_dec, latent, c_scale, kv_off, max_len, k, out_idx=None, out_scores=None,
                          flags=LI_LATENT_FP16, ws=None, stream=None):
    """LatentIndex group scan + per-layer top-k.  q [B,G,H,Dh] bf16, w [B,G,H] fp32,
    w_dec [G,Dc,H*Dh] bf16, latent [n_tok,Dc] bf16.  Returns out_idx [B,G,k]."""
    B, G, H, Dh = q.shape
    n_tok, Dc = latent.shape
    if out_idx is None:
        out_idx = torch.empty((B, G, k), dtype=torch.int32, device=q.device)
    L = lib()
    need = L.li_latent_score_group_ws(B, n_tok, max_len, G, H, Dc, k, int(out_scores is not None))
    wst, wsb = _workspace(need, q.device, ws)
    _check(L.li_latent_score_group(_ptr(q), _dt(q), _ptr(w), _ptr(w_dec), _dt(w_dec), _ptr(latent), _dt(latent),
                                   _ptr(c_scale), _ptr(kv_off), B, n_tok, max_len, G, H, Dh, Dc, k, _ptr(out_idx),
                                   _ptr(out_scores), flags, _ptr(wst), wsb, _stream(stream)))
    return out_idx


def li_hs_refine(cand_idx, q, w, w_dec, latent, c_scale, kv_off, k, out_idx=None, out_scores=None,
                 flags=LI_LATENT_FP16, ws=None, stream=None):
    """HS follower rescoring.  cand_idx [B,C] int32 (ascending, -1 padded),
    q [B,Gf,H,Dh] bf16, w [B,Gf,H], w_dec [Gf,Dc,H*Dh] bf16, latent [n_tok,Dc]
    bf16.  Returns out_idx [B,Gf,k] token positions."""
    B, Cn = cand_idx.shape
    _, Gf, H, Dh = q.shape
    Dc = latent.shape[1]
    if out_idx is None:
        out_idx = torch.empty((B, Gf, k), dtype=torch.int32, device=q.device)
    L = lib()
    need = L.li_hs_refine_ws(B, Cn, Gf, H, Dc, k, int(out_scores is not None))
    wst, wsb = _workspace(need, q.device, ws)
    _check(L.li_hs_refine(_ptr(cand_idx), Cn, _ptr(q), _dt(q), _ptr(w), _ptr(w_dec), _dt(w_dec), _ptr(latent),
                          _dt(latent), _ptr(c_scale), _ptr(kv_off), B, Gf, H, Dh, Dc, k, _ptr(out_idx),
                          _ptr(out_scores), flags, _ptr(wst), wsb, _stream(stream)))
    return out_idx


def li_latent_append(h, w_enc, dst_row, latent, c_scale=None, ws=None, stream=None):
    """Latent-cache append: latent[dst_row[m]] = quantised(w_enc @ h[m]) in place.
    h [M,d_model] bf16, w_enc [Dc,d_model] bf16, dst_row [M] int64, latent
    [n_tok,Dc] bf16, or float8_e4m3fn with c_scale [n_tok,Dc/128] fp32 (block
    scales, written too).  Returns latent."""
    M, d_model = h.shape
    Dc = w_enc.shape[0]
    n_tok = latent.shape[0]
    L = lib()
    c_dt = _dt(latent)
    need = L.li_latent_append_ws(M, d_model, Dc, c_dt)
    wst, wsb = _workspace(need, latent.device, ws)
    _check(L.li_latent_append(_ptr(h), _dt(h), _ptr(w_enc), _dt(w_enc), _ptr(dst_row), M, d_model, Dc, _ptr(latent),
                              c_dt, _ptr(c_scale), n_tok, _ptr(wst), wsb, _stream(stream)))
    return latent


def li_sparse_attention(q, kv, idx, kv_off, scale, out=None, ws=None, stream=None):
    """Attention over selected rows.  q [B,H,576] bf16, kv [n_tok,576] bf16,
    idx [B,k] int32 (-1 padded), kv_off [B+1] int64.  Returns out [B,H,512] fp32."""
    B, H, Dk = q.shape
    k = idx.shape[1]
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=q.device)
    L = lib()
    need = L.li_sparse_attention_ws(B, H, k)
    wst, wsb = _workspace(need, q.device, ws)
    _check(L.li_sparse_attention(_ptr(q), _dt(q), _ptr(kv), _dt(kv), _ptr(idx), _ptr(kv_off), B, kv.shape[0], H, Dk,
                                 512, k, float(scale), _ptr(out), _ptr(wst), wsb, _stream(stream)))
    return out


def li_indexcache_plan(n_layers, retain_every=1, roles=None):
    """IndexCache schedule (host only): returns (number of F layers, src) where
    src[l] is the layer whose selection layer l attends.  roles: optional
    sequence of 1 (F) / 0 (S); otherwise every retain_every-th layer is F."""
    import ctypes
    src = (ctypes.c_int32 * n_layers)()
    r = None if roles is None else (ctypes.c_uint8 * n_layers)(*[1 if x else 0 for x in roles])
    n = lib().li_indexcache_plan(r, n_layers, retain_every, src)
    if n < 0:
        _check(-n)
    return n, list(src)


def li_topk(scores, k, row_len=None, n=None, out_idx=None, ws=None, stream=None):
    """Row-wise top-k of scores [rows, stride] fp32; row_len [rows] int32 or None."""
    rows, stride = scores.shape
    n = stride if n is None else n
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    L = lib()
    need = L.li_topk_ws(rows, n, k)
    wst, wsb = _workspace(need, scores.device, ws)
    _check(L.li_topk(_ptr(scores), stride, _ptr(row_len), rows, n, k, _ptr(out_idx), _ptr(wst), wsb,
                     _stream(stream)))
    return out_idx


def li_read_probe(buf, sink, stream=None):
    """Stream every byte of the CUDA tensor buf once (measurement aid);
    sink is a [LI_READ_PROBE_SINK_WORDS] int32 CUDA tensor."""
    _check(lib().li_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def li_mfma_probe(form, random_operands, iters, sink, clk, stream=None):
    """Run the matrix-core rate probe (measurement aid): form LI_MFMA_PROBE_*,
    constant (False) or random (True) operands; sink is a
    [LI_MFMA_PROBE_SINK_WORDS] float32 and clk a [LI_MFMA_PROBE_CLOCK_WORDS]
    int32 CUDA tensor."""
    _check(lib().li_mfma_probe(int(form), 1 if random_operands else 0, int(iters), _ptr(sink), _ptr(clk),
                               _stream(stream)))


def li_trace_events(events, capacity):
    """Switch the measurement hook on (a ctypes array of hipEvent_t) or off (None, 0)."""
    lib().li_trace_events(events, capacity)


def li_trace_count():
    return lib().li_trace_count()
