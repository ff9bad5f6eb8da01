"""CPU oracle for the lightning-indexer scan: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg import this package.  It wraps ``liboracle.so`` (plain C, double
precision, direct loops plus a full sort for top-k; see ``oracle.c`` for the
definition and its sources) and shares no code with the HIP library.

Arrays are numpy.  Element types are named by strings: "bf16" and "fp16"
arrays are raw uint16 bit patterns, "fp8_e4m3" arrays are raw uint8 bytes
(OCP E4M3FN), "fp32" arrays are float32.

Parity of every function here is pinned by ``tests/test_oracle_pins.py``.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_CODES = {"bf16": 0, "fp8_e4m3": 1, "fp16": 2, "fp32": 3}
_RAW = {"bf16": np.uint16, "fp8_e4m3": np.uint8, "fp16": np.uint16, "fp32": np.float32}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = C.CDLL(_build.LIB)
        vp, i32, i64, dp = C.c_void_p, C.c_int, C.c_int64, C.c_void_p
        _lib.oracle_decode_element.restype = C.c_double
        _lib.oracle_decode_element.argtypes = [vp, i32, i64]
        _lib.oracle_topk.argtypes = [vp, i64, vp, i32, i32, vp]
        _lib.oracle_index_decode.argtypes = [vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, dp, dp]
        _lib.oracle_index_prefill.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, dp, dp]
        _lib.oracle_latent_absorb.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, dp]
        _lib.oracle_latent_score_group.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, dp, dp]
        _lib.oracle_latent_reconstruct_scores.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, dp]
        _lib.oracle_hs_refine.argtypes = [vp, i32, vp, i32, vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, dp, dp]
        _lib.oracle_latent_append.argtypes = [vp, i32, vp, i32, vp, i32, i32, i32, vp, i32, vp, i64, dp]
        _lib.oracle_encode_e4m3.restype = C.c_uint8
        _lib.oracle_encode_e4m3.argtypes = [C.c_double]
        _lib.oracle_sparse_attention.argtypes = [vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, C.c_double, dp, dp]
        _lib.oracle_encode_bf16.restype = C.c_uint16
        _lib.oracle_encode_bf16.argtypes = [C.c_double]
        for f in ("oracle_topk", "oracle_index_decode", "oracle_index_prefill", "oracle_latent_absorb",
                  "oracle_latent_score_group", "oracle_latent_reconstruct_scores", "oracle_hs_refine",
                  "oracle_latent_append", "oracle_sparse_attention"):
            getattr(_lib, f).restype = C.c_int
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dt):
    a = np.ascontiguousarray(a)
    want = _RAW[dt]
    if a.dtype != want:
        raise TypeError(f"{dt} data must be a {np.dtype(want).name} array, got {a.dtype}")
    return a


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def decode_element(raw, dt):
    """Decode every element of a raw array of type ``dt`` to float64."""
    raw = _arr(raw, dt).reshape(-1)
    L = lib()
    return np.array([L.oracle_decode_element(_p(raw), _CODES[dt], i) for i in range(raw.size)])


def topk(scores, lens, k, stride=None):
    """Row-wise top-k of float64 scores [rows][stride]; lens[r] values count."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    rows = s.shape[0]
    stride = s.shape[1] if stride is None else stride
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    out = np.empty((rows, k), dtype=np.int32)
    _check(lib().oracle_topk(_p(s), stride, _p(lens), rows, k, _p(out)), "oracle_topk")
    return out


def index_decode(q, q_dt, w, kc, k_dt, k_scale, kv_off, H, D, k, want_scores=True):
    q, kc = _arr(q, q_dt), _arr(kc, k_dt)
    w, k_scale = _f32(w), _f32(k_scale)
    kv_off = np.ascontiguousarray(kv_off, dtype=np.int64)
    B = kv_off.size - 1
    n_tok = int(kv_off[-1])
    idx = np.empty((B, k), dtype=np.int32)
    sc = np.empty(n_tok, dtype=np.float64) if want_scores else None
    ab = np.empty(n_tok, dtype=np.float64) if want_scores else None
    rc = lib().oracle_index_decode(_p(q), _CODES[q_dt], _p(w), _p(kc), _CODES[k_dt], _p(k_scale),
                                   _p(kv_off), B, H, D, k, _p(idx), _p(sc), _p(ab))
    _check(rc, "oracle_index_decode")
    return idx, sc, ab


def index_prefill(q, q_dt, q_scale, w, kc, k_dt, k_scale, T, L, qpos0, H, D, k, want_scores=True):
    q, kc = _arr(q, q_dt), _arr(kc, k_dt)
    w, q_scale, k_scale = _f32(w), _f32(q_scale), _f32(k_scale)
    idx = np.empty((T, k), dtype=np.int32)
    sc = np.empty((T, L), dtype=np.float64) if want_scores else None
    ab = np.empty((T, L), dtype=np.float64) if want_scores else None
    rc = lib().oracle_index_prefill(_p(q), _CODES[q_dt], _p(q_scale), _p(w), _p(kc), _CODES[k_dt],
                                    _p(k_scale), T, L, qpos0, H, D, k, _p(idx), _p(sc), _p(ab))
    _check(rc, "oracle_index_prefill")
    return idx, sc, ab


def latent_absorb(q, q_dt, w_dec, w_dt, B, G, H, Dh, Dc):
    q, w_dec = _arr(q, q_dt), _arr(w_dec, w_dt)
    out = np.empty((B, G, H, Dc), dtype=np.float64)
    _check(lib().oracle_latent_absorb(_p(q), _CODES[q_dt], _p(w_dec), _CODES[w_dt], B, G, H, Dh, Dc, _p(out)),
           "oracle_latent_absorb")
    return out


def latent_score_group(q, q_dt, w, w_dec, w_dt, latent, c_dt, c_scale, kv_off, G, H, Dh, Dc, k,
                       want_scores=True, c_blocks=1):
    """c_scale: [n_tok] per-row scales, or [n_tok][c_blocks] with c_blocks = ceil(Dc / 128) (one per
    128-value block, the last one shorter when Dc is not a multiple of 128)."""
    q, w_dec, latent = _arr(q, q_dt), _arr(w_dec, w_dt), _arr(latent, c_dt)
    w, c_scale = _f32(w), _f32(c_scale)
    kv_off = np.ascontiguousarray(kv_off, dtype=np.int64)
    B = kv_off.size - 1
    n_tok = int(kv_off[-1])
    idx = np.empty((B, G, k), dtype=np.int32)
    sc = np.empty((G, n_tok), dtype=np.float64) if want_scores else None
    ab = np.empty((G, n_tok), dtype=np.float64) if want_scores else None
    rc = lib().oracle_latent_score_group(_p(q), _CODES[q_dt], _p(w), _p(w_dec), _CODES[w_dt], _p(latent),
                                         _CODES[c_dt], _p(c_scale), c_blocks, _p(kv_off), B, G, H, Dh, Dc, k,
                                         _p(idx), _p(sc), _p(ab))
    _check(rc, "oracle_latent_score_group")
    return idx, sc, ab


def latent_reconstruct_scores(q, q_dt, w, w_dec, w_dt, latent, c_dt, c_scale, kv_off, G, H, Dh, Dc, c_blocks=1):
    q, w_dec, latent = _arr(q, q_dt), _arr(w_dec, w_dt), _arr(latent, c_dt)
    w, c_scale = _f32(w), _f32(c_scale)
    kv_off = np.ascontiguousarray(kv_off, dtype=np.int64)
    B = kv_off.size - 1
    sc = np.empty((G, int(kv_off[-1])), dtype=np.float64)
    rc = lib().oracle_latent_reconstruct_scores(_p(q), _CODES[q_dt], _p(w), _p(w_dec), _CODES[w_dt],
                                                _p(latent), _CODES[c_dt], _p(c_scale), c_blocks, _p(kv_off), B, G, H,
                                                Dh, Dc, _p(sc))
    _check(rc, "oracle_latent_reconstruct_scores")
    return sc


def hs_refine(cand_idx, q, q_dt, w, w_dec, w_dt, latent, c_dt, c_scale, kv_off, Gf, H, Dh, Dc, k,
              want_scores=True, c_blocks=1):
    cand_idx = np.ascontiguousarray(cand_idx, dtype=np.int32)
    q, w_dec, latent = _arr(q, q_dt), _arr(w_dec, w_dt), _arr(latent, c_dt)
    w, c_scale = _f32(w), _f32(c_scale)
    kv_off = np.ascontiguousarray(kv_off, dtype=np.int64)
    B, Cn = cand_idx.shape
    idx = np.empty((B, Gf, k), dtype=np.int32)
    sc = np.full((B, Gf, Cn), np.nan) if want_scores else None
    ab = np.full((B, Gf, Cn), np.nan) if want_scores else None
    rc = lib().oracle_hs_refine(_p(cand_idx), Cn, _p(q), _CODES[q_dt], _p(w), _p(w_dec), _CODES[w_dt],
                                _p(latent), _CODES[c_dt], _p(c_scale), c_blocks, _p(kv_off), B, Gf, H, Dh, Dc, k,
                                _p(idx), _p(sc), _p(ab))
    _check(rc, "oracle_hs_refine")
    return idx, sc, ab


def encode_bf16(v):
    """The bfloat16 code (uint16) nearest to float v, ties to even."""
    return int(lib().oracle_encode_bf16(float(v)))


def encode_e4m3(v):
    """The OCP E4M3FN code (uint8) nearest to float v, ties to even, saturating at 448."""
    return int(lib().oracle_encode_e4m3(float(v)))


def latent_append(h, h_dt, w_enc, w_dt, dst_row, latent, c_scale=None):
    """Latent-cache append: c[b][d] = sum_i h[b][i] * w_enc[d][i] (fp64), stored
    at row dst_row[b] of a copy of `latent`: [n_tok][Dc] raw bf16 (uint16), or
    with c_scale ([n_tok][ceil(Dc/128)] float32) E4M3 codes (uint8) with per-block
    scales.  Returns (new latent, exact sums [B][Dc]) or, for fp8,
    (new latent, new scales, exact sums)."""
    h = _arr(h, h_dt)
    w_enc = _arr(w_enc, w_dt)
    B, d_model = h.shape
    Dc = w_enc.shape[0]
    assert w_enc.shape == (Dc, d_model)
    fp8 = c_scale is not None
    out = np.array(latent, dtype=np.uint8 if fp8 else np.uint16, copy=True)
    sc = np.array(c_scale, dtype=np.float32, copy=True) if fp8 else None
    n_tok = out.shape[0]
    dst = np.ascontiguousarray(dst_row, dtype=np.int64)
    exact = np.zeros((B, Dc), np.float64)
    _check(lib().oracle_latent_append(_p(h), _CODES[h_dt], _p(w_enc), _CODES[w_dt], _p(dst), B, d_model, Dc,
                                      _p(out), _CODES["fp8_e4m3" if fp8 else "bf16"], _p(sc), n_tok, _p(exact)),
           "oracle_latent_append")
    return (out, sc, exact) if fp8 else (out, exact)


def sparse_attention(q, q_dt, kv, kv_dt, idx, kv_off, scale, Dv):
    """Attention of each request's heads over its selected cache rows.
    q [B][H][Dk], kv [n_tok][Dk], idx [B][K] int32 (-1 = none), kv_off [B+1].
    Returns (out [B][H][Dv] fp64, mag [B][H][Dv] = sum p|v| / sum p)."""
    q = _arr(q, q_dt)
    kv = _arr(kv, kv_dt)
    B, H, Dk = q.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    K = idx.shape[1] if idx.ndim == 2 else 0
    off = np.ascontiguousarray(kv_off, dtype=np.int64)
    out = np.zeros((B, H, Dv), np.float64)
    mag = np.zeros((B, H, Dv), np.float64)
    _check(lib().oracle_sparse_attention(_p(q), _CODES[q_dt], _p(kv), _CODES[kv_dt], _p(idx), _p(off), B, H, K, Dk,
                                          Dv, float(scale), _p(out), _p(mag)), "oracle_sparse_attention")
    return out, mag
