"""Seeded synthetic inputs shaped like the lightning-indexer workloads.

This module is shared by the tests, the benchmark, the smoke check and the
CPU oracle's callers.  It holds none of the method's arithmetic: it only
draws random numbers (numpy PCG64, fixed seeds, fixed draw order) and encodes
them into the storage types the library takes (bf16 and OCP FP8 E4M3FN bit
patterns, via torch's round-to-nearest-even casts; fp8 saturates at +-448).

Workload shapes (64 indexer heads x 128 dims per key, k = 2048) follow
"LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for Sparse
Attention", Table 5, and the k = 2,048 selection budget of "IndexCache:
Cross-Layer Index Reuse for Sparse Attention", Symbol Map.  The pages state no
value distributions; the recipes below are the ones documented for this
library (integer-valued bf16 for the exact case, N(0,1) fp8 keys with U[0.5,2)
per-token scales, N(0, 1/64) head weights, N(0,1) bf16 latents, N(0, 1/Dc)
decoders).

Draw order inside one workload: lengths, q, w, K, sigma, latent, W.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0


def encode_bf16(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def encode_fp8(x) -> np.ndarray:
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode(x, dt) -> np.ndarray:
    if dt == "bf16":
        return encode_bf16(x)
    if dt == "fp8_e4m3":
        return encode_fp8(x)
    if dt == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dt)


@dataclass
class Decode:
    """One decode step: B requests, one query token each, ragged key cache."""
    q: np.ndarray            # [B][H][D] bf16 bits
    w: np.ndarray            # [B][H] float32
    kc: np.ndarray           # [n_tok][D] raw (k_dt)
    k_scale: Optional[np.ndarray]  # [n_tok] float32 or None
    kv_off: np.ndarray       # [B+1] int64
    H: int
    D: int
    k: int
    q_dt: str = "bf16"
    k_dt: str = "fp8_e4m3"
    name: str = ""

    @property
    def B(self):
        return self.kv_off.size - 1

    @property
    def n_tok(self):
        return int(self.kv_off[-1])

    @property
    def lens(self):
        return np.diff(self.kv_off)


@dataclass
class Prefill:
    """One prefill chunk: T new query tokens, causal over an L-token cache."""
    q: np.ndarray            # [T][H][D] raw (q_dt)
    q_scale: Optional[np.ndarray]  # [T] float32 or None
    w: np.ndarray            # [T][H] float32
    kc: np.ndarray           # [L][D] raw (k_dt)
    k_scale: Optional[np.ndarray]  # [L] float32 or None
    T: int
    L: int
    qpos0: int
    H: int
    D: int
    k: int
    q_dt: str = "fp8_e4m3"
    k_dt: str = "fp8_e4m3"
    name: str = ""


@dataclass
class Latent:
    """A LatentIndex group: G layers over one shared latent cache."""
    q: np.ndarray            # [B][G][H][Dh] bf16 bits
    w: np.ndarray            # [B][G][H] float32
    w_dec: np.ndarray        # [G][Dc][H*Dh] bf16 bits
    latent: np.ndarray       # [n_tok][Dc] bf16 bits, or fp8 codes (c_dt "fp8_e4m3")
    c_scale: Optional[np.ndarray]  # [n_tok] row scales, or [n_tok][Dc/128] block scales (fp8)
    kv_off: np.ndarray
    G: int
    H: int
    Dh: int
    Dc: int
    k: int
    q_dt: str = "bf16"
    w_dt: str = "bf16"
    c_dt: str = "bf16"
    name: str = ""

    @property
    def B(self):
        return self.kv_off.size - 1

    @property
    def n_tok(self):
        return int(self.kv_off[-1])

    @property
    def c_blocks(self):
        return 1 if self.c_scale is None or self.c_scale.ndim == 1 else int(self.c_scale.shape[1])


def quantize_fp8_blocks(values, block=128):
    """fp8 storage of a latent: per row, one fp32 scale per `block` values
    counted from the row's start (a width that is not a multiple of `block`
    ends in a shorter block) -- the block's largest magnitude / 448, or 1 for
    an all-zero block -- and the values / scale as OCP E4M3 codes (round to
    nearest even)."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    n, d = v.shape
    nb = (d + block - 1) // block
    sc = np.empty((n, nb), np.float32)
    scaled = np.empty_like(v)
    for j in range(nb):
        blk = v[:, j * block:(j + 1) * block]
        s = (np.abs(blk).max(axis=1) / np.float32(FP8_MAX)).astype(np.float32)
        s[s == 0] = 1.0
        sc[:, j] = s
        scaled[:, j * block:(j + 1) * block] = blk / s[:, None]
    return encode_fp8(scaled), sc


def latent_to_fp8(x):
    """The same workload with its latent stored as fp8 with 128-value block scales
    (the bf16 values requantised)."""
    vals = torch.from_numpy(x.latent.view(np.int16)).view(torch.bfloat16).float().numpy()
    codes, sc = quantize_fp8_blocks(vals)
    x.latent, x.c_scale, x.c_dt = codes, sc, "fp8_e4m3"
    x.name = x.name.replace("latent_", "latent_fp8_") if x.name else x.name
    return x


@dataclass
class HS:
    """Hierarchical selection: fp8 anchor decode with k = C, then Gf followers."""
    anchor: Decode
    followers: Latent        # G = Gf; shares kv_off with the anchor
    C: int
    name: str = ""


def _draw_lens(rng, lens):
    """lens is either explicit per-request lengths or ("uniform", lo, hi, B):
    B lengths uniform over the integers lo..hi, drawn first from the stream."""
    if isinstance(lens, tuple) and lens and lens[0] == "uniform":
        _, lo, hi, B = lens
        return rng.integers(lo, hi + 1, size=B).astype(np.int64)
    return np.asarray(lens, dtype=np.int64)


def _offsets(lens):
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return off


def make_decode(seed, lens, H=64, D=128, k=2048, k_dt="fp8_e4m3", dist="normal", scales=True,
                name="") -> Decode:
    """Decode inputs.  dist="normal": q ~ N(0,1) -> bf16, K ~ N(0,1) -> k_dt,
    w ~ N(0, 1/64), sigma ~ U[0.5, 2).  dist="int": q, K integers uniform on
    [-3, 3] and w integers uniform on [-2, 2] (exact in fp32), no scales."""
    rng = np.random.default_rng(seed)
    lens = _draw_lens(rng, lens)
    B = lens.size
    off = _offsets(lens)
    n = int(off[-1])
    if dist == "int":
        q = rng.integers(-3, 4, size=(B, H, D)).astype(np.float32)
        w = rng.integers(-2, 3, size=(B, H)).astype(np.float32)
        kf = rng.integers(-3, 4, size=(n, D)).astype(np.float32)
        sc = None
    else:
        q = rng.standard_normal((B, H, D), dtype=np.float32)
        w = (rng.standard_normal((B, H), dtype=np.float32) * np.float32(0.125)).astype(np.float32)
        kf = rng.standard_normal((n, D), dtype=np.float32)
        sc = rng.uniform(0.5, 2.0, size=n).astype(np.float32) if scales else None
    return Decode(q=encode_bf16(q), w=w, kc=encode(kf, k_dt), k_scale=sc, kv_off=off, H=H, D=D, k=k,
                  k_dt=k_dt, name=name)


def make_prefill(seed, T, L, H=64, D=128, k=2048, qpos0=None, name="") -> Prefill:
    """Prefill inputs: q_hat, K_hat ~ N(0,1) -> fp8, sigma_q, sigma_k ~ U[0.5, 2),
    w ~ N(0, 1/64) per query token.  The new tokens are the last T of the cache."""
    rng = np.random.default_rng(seed)
    qpos0 = L - T if qpos0 is None else qpos0
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    w = (rng.standard_normal((T, H), dtype=np.float32) * np.float32(0.125)).astype(np.float32)
    kf = rng.standard_normal((L, D), dtype=np.float32)
    ks = rng.uniform(0.5, 2.0, size=L).astype(np.float32)
    qs = rng.uniform(0.5, 2.0, size=T).astype(np.float32)
    return Prefill(q=encode_fp8(q), q_scale=qs, w=w, kc=encode_fp8(kf), k_scale=ks, T=T, L=L, qpos0=qpos0,
                   H=H, D=D, k=k, name=name)


def _latent_parts(rng, B, G, H, Dh, Dc, n):
    q = rng.standard_normal((B, G, H, Dh), dtype=np.float32)
    w = (rng.standard_normal((B, G, H), dtype=np.float32) * np.float32(0.125)).astype(np.float32)
    lat = rng.standard_normal((n, Dc), dtype=np.float32)
    W = (rng.standard_normal((G, Dc, H * Dh), dtype=np.float32) * np.float32(1.0 / np.sqrt(Dc))).astype(np.float32)
    return encode_bf16(q), w, encode_bf16(lat), encode_bf16(W)


def make_latent(seed, lens, G=4, H=64, Dh=128, Dc=256, k=2048, name="") -> Latent:
    """LatentIndex group inputs: q ~ N(0,1) -> bf16, w ~ N(0, 1/64), latent ~
    N(0,1) -> bf16, W_l ~ N(0, 1/Dc) -> bf16, no latent scales."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    off = _offsets(lens)
    q, w, lat, W = _latent_parts(rng, lens.size, G, H, Dh, Dc, int(off[-1]))
    return Latent(q=q, w=w, w_dec=W, latent=lat, c_scale=None, kv_off=off, G=G, H=H, Dh=Dh, Dc=Dc, k=k,
                  name=name)


def make_hs(seed, lens, C=8192, Gf=3, H=64, D=128, Dc=256, k=2048, name="") -> HS:
    """HS inputs: an fp8 anchor decode (as make_decode) and Gf latent followers
    (as make_latent) over the same requests."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B = lens.size
    off = _offsets(lens)
    n = int(off[-1])
    q = rng.standard_normal((B, H, D), dtype=np.float32)
    w = (rng.standard_normal((B, H), dtype=np.float32) * np.float32(0.125)).astype(np.float32)
    kf = rng.standard_normal((n, D), dtype=np.float32)
    sc = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
    anchor = Decode(q=encode_bf16(q), w=w, kc=encode_fp8(kf), k_scale=sc, kv_off=off, H=H, D=D, k=C,
                    name=name + "/anchor")
    del kf
    fq, fw, lat, W = _latent_parts(rng, B, Gf, H, D, Dc, n)
    fol = Latent(q=fq, w=fw, w_dec=W, latent=lat, c_scale=None, kv_off=off, G=Gf, H=H, Dh=D, Dc=Dc, k=k,
                 name=name + "/followers")
    return HS(anchor=anchor, followers=fol, C=C, name=name)


# ---- the five workloads (seed = 1000 + workload number) ------------------------

@dataclass
class Append:
    """Latent-cache append: M new tokens' hidden states written into a ragged
    latent cache, request b's j-th new token at row kv_off[b] + old_b + j."""
    h: np.ndarray            # [M][d_model] bf16 bits
    w_enc: np.ndarray        # [Dc][d_model] bf16 bits
    dst_row: np.ndarray      # [M] int64
    kv_off: np.ndarray       # [B+1] int64 over each request's old + new length
    n_tok: int
    d_model: int
    Dc: int
    name: str = ""

    @property
    def M(self):
        return int(self.dst_row.size)


def make_append(seed, old_lens, new_lens, d_model=7168, Dc=256, dist="normal", name="") -> Append:
    """Append inputs.  dist "normal": h ~ N(0,1) -> bf16 and W_enc ~
    N(0, 1/d_model) -> bf16 (latent entries of unit scale); "int": both
    integers uniform on -3..3 (every sum exact in fp32).  The cache row of
    each new token follows its request's old tokens.  The pages give no
    hidden size or encoder distribution: d_model = 7168 is a stand-in."""
    rng = np.random.default_rng(seed)
    old = np.asarray(old_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    off = _offsets(old + new)
    dst = np.concatenate([off[b] + old[b] + np.arange(new[b], dtype=np.int64) for b in range(old.size)] +
                         [np.zeros(0, np.int64)])
    M = int(dst.size)
    if dist == "int":
        h = rng.integers(-3, 4, size=(M, d_model)).astype(np.float32)
        W = rng.integers(-3, 4, size=(Dc, d_model)).astype(np.float32)
    else:
        h = rng.standard_normal((M, d_model), dtype=np.float32)
        W = (rng.standard_normal((Dc, d_model), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_model))).astype(
            np.float32)
    return Append(h=encode_bf16(h), w_enc=encode_bf16(W), dst_row=dst, kv_off=off, n_tok=int(off[-1]),
                  d_model=d_model, Dc=Dc, name=name)


def append_decode() -> Append:
    """One decode step's append for the LatentIndex group: B = 16 requests at
    L = 131072, one new token each, Dc = 256."""
    return make_append(1006, [131072] * 16, [1] * 16, name="append_decode_B16_L131072_d7168_Dc256")


def append_prefill() -> Append:
    """A prefill chunk's append: 4096 new tokens ending a 65536-token cache, Dc = 256."""
    return make_append(1007, [65536 - 4096], [4096], name="append_prefill_T4096_L65536_d7168_Dc256")


@dataclass
class Attention:
    """Sparse attention over selected rows: B requests, H heads, a latent KV
    cache of Dk = 576 values per token, idx [B][k] ascending, -1 padded."""
    q: np.ndarray            # [B][H][576] bf16 bits
    kv: Optional[np.ndarray]  # [n_tok][576] bf16 bits (None: drawn on the device)
    idx: np.ndarray          # [B][k] int32
    kv_off: np.ndarray       # [B+1] int64
    H: int
    k: int
    scale: float
    seed: int = 0
    name: str = ""

    @property
    def B(self):
        return int(self.kv_off.size - 1)

    @property
    def n_tok(self):
        return int(self.kv_off[-1])


def _selection(rng, lens, k):
    idx = np.full((len(lens), k), -1, np.int32)
    for b, n in enumerate(lens):
        m = int(min(n, k))
        if m:
            idx[b, :m] = np.sort(rng.choice(int(n), m, replace=False))
    return idx


def make_attention(seed, lens, H=64, k=2048, device_kv=False, name="") -> Attention:
    """q ~ N(0,1) and kv ~ N(0,1) -> bf16; each request selects min(L_b, k)
    distinct positions uniformly, ascending, -1 padded; scale 1/sqrt(192) (a
    128 + 64-dim query-key head).  device_kv: the cache is drawn later on the
    GPU by device_kv_cache(), for caches too large to draw on the host."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    off = _offsets(lens)
    q = rng.standard_normal((lens.size, H, 576), dtype=np.float32)
    idx = _selection(rng, lens, k)
    kv = None if device_kv else encode_bf16(rng.standard_normal((int(off[-1]), 576), dtype=np.float32))
    return Attention(q=encode_bf16(q), kv=kv, idx=idx, kv_off=off, H=H, k=k, scale=float(1.0 / np.sqrt(192.0)),
                     seed=seed, name=name)


def device_kv_cache(x: Attention):
    """The cache of a device_kv workload: N(0,1) -> bf16 from a torch generator
    on the current GPU, seeded by the workload's seed."""
    g = torch.Generator(device="cuda")
    g.manual_seed(x.seed)
    return torch.randn((x.n_tok, 576), generator=g, device="cuda").to(torch.bfloat16)


def attention_decode() -> Attention:
    """Sparse attention of one decode step after the indexer: B = 16 requests at
    L = 131072, 128 heads, k = 2048 selected rows each."""
    return make_attention(1008, [131072] * 16, H=128, device_kv=True, name="attention_B16_L131072_H128_k2048")


def cfg1() -> Decode:
    """Single decode query, L = 4096, integer-valued bf16 q and K, integer w."""
    return make_decode(1001, [4096], k_dt="bf16", dist="int", name="decode_int_L4096")


def cfg2() -> Decode:
    """Batched decode, B = 32, ragged L_b ~ U{8192..32768}, fp8 keys + scales."""
    return make_decode(1002, ("uniform", 8192, 32768, 32), name="decode_fp8_B32_ragged8K-32K")


def decode_sweep(L, B=32, seed=None) -> Decode:
    """Batched decode at a fixed context L (cfg2 distributions)."""
    return make_decode(2000 + L // 1024 if seed is None else seed, [L] * B, name=f"decode_fp8_B{B}_L{L}")


def cfg3() -> Prefill:
    """Prefill chunk: T = 4096 new tokens, causal cache L = 65536, fp8 q and K."""
    return make_prefill(1003, 4096, 65536, name="prefill_fp8_T4096_L65536")


def cfg4() -> Latent:
    """LatentIndex group decode: G = 4, B = 16, L = 131072, Dc = 256, bf16."""
    return make_latent(1004, [131072] * 16, name="latent_G4_B16_L131072")


def cfg5() -> HS:
    """HS decode: fp8 anchor top-8192 over L = 131072, 3 latent followers, B = 16."""
    return make_hs(1005, [131072] * 16, name="hs_B16_L131072_C8192_F3")
