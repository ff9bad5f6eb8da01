// LatentIndex and HS kernels on gfx950 ("LatentIndex: Cross-Layer Sharing with
// Layer-Specific Selection for Sparse Attention", Abstract and Figure 1).
//
// A group of G layers shares one latent cache c (one Dc-dim row per token).
// Layer l's key decoder W_l ([Dc][H*Dh]; head h's key is
// k[j] = sum_c W_l[c][h*Dh + j] c[c]) is absorbed into the query,
//   qt[l][h][c] = sum_j W_l[c][h*Dh + j] q[l][h][j],
// so every historical token is scored straight from the shared cache,
//   S_l[s] = c_scale[s] * sum_h w[l][h] * ReLU(qt[l][h] . c_s),
// without reconstructing per-layer keys.  HS followers do the same over the
// anchor's candidate rows only.
//
// latent_absorb: one workgroup per (layer, head); fp32 accumulation; the
//   result is stored as an fp16 MFMA operand after scaling the row by a power
//   of two that puts its largest magnitude in [2^14, 2^15) (exact), with the
//   inverse folded into the head weight.  fp16 keeps 11 significant bits,
//   which is what the score tolerance needs; bf16 (8 bits) would not.
// latent_score: one pass over the latent rows for all layers of the group.  A
//   workgroup stages 32 latent rows at a time through LDS, converting bf16 ->
//   fp16 once (exact in fp16 range) and writing them in MFMA-fragment order;
//   each of its four waves holds one layer's 64 x Dc absorbed query in
//   registers and runs v_mfma_f32_32x32x16_f16 against the shared tile, then
//   the same ReLU-weighted head reduction as the native scan.  The gather
//   variant (HS) reads rows kv_off[b] + cand[b][j] instead of contiguous ones.
//   The contiguous variant also builds each (request, layer) row's level-0
//   selection histogram in LDS and stores it as the workgroup's partial.
#include <math.h>

#include "li_device.h"
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kAbsB = 32;  // requests per absorb pass

__global__ __launch_bounds__(256) void latent_absorb_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ w_dec,
    int B, int G, int H, int Dc, uint16_t* __restrict__ qt16, float* __restrict__ wsc) {
  constexpr int Dh = 128;
  __shared__ float qs[kAbsB][Dh];
  __shared__ float red[kAbsB][4];
  const int l = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int c = threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* wrow = w_dec + ((int64_t)l * Dc + (c < Dc ? c : 0)) * (int64_t)H * Dh + (int64_t)h * Dh;

  for (int b0 = 0; b0 < B; b0 += kAbsB) {
    const int nb = (B - b0) < kAbsB ? (B - b0) : kAbsB;
    for (int i = threadIdx.x; i < kAbsB * Dh; i += 256) {
      const int bi = i / Dh, j = i - (i / Dh) * Dh;
      float v = 0.0f;
      if (bi < nb) {
        const uint16_t raw = q[(((int64_t)(b0 + bi) * G + l) * H + h) * Dh + j];
        v = __builtin_bit_cast(float, (uint32_t)raw << 16);
      }
      qs[bi][j] = v;
    }
    __syncthreads();
    float acc[kAbsB];
#pragma unroll
    for (int bi = 0; bi < kAbsB; ++bi) acc[bi] = 0.0f;
    if (c < Dc) {
#pragma unroll 1
      for (int j0 = 0; j0 < Dh; j0 += 8) {
        const i32x4 v = ld16(wrow + j0);
        const int parts[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int word = parts[e >> 1];
          const float wv = __builtin_bit_cast(float, (e & 1) ? (word & (int)0xFFFF0000u) : (word << 16));
#pragma unroll
          for (int bi = 0; bi < kAbsB; ++bi) acc[bi] = fmaf(wv, qs[bi][j0 + e], acc[bi]);
        }
      }
    }
#pragma unroll
    for (int bi = 0; bi < kAbsB; ++bi) {
      const float m = wave_max(c < Dc ? fabsf(acc[bi]) : 0.0f);
      if (lane == 0) red[bi][wave] = m;
    }
    __syncthreads();
    for (int bi = 0; bi < nb; ++bi) {
      const float mx = fmaxf(fmaxf(red[bi][0], red[bi][1]), fmaxf(red[bi][2], red[bi][3]));
      int E = 0;
      if (mx > 0.0f) frexpf(mx, &E);
      const int e = mx > 0.0f ? 15 - E : 0;  // mx * 2^e in [2^14, 2^15)
      const int64_t rowi = ((int64_t)(b0 + bi) * G + l) * H + h;
      if (c < Dc) {
        const _Float16 hv = (_Float16)ldexpf(acc[bi], e);
        qt16[rowi * Dc + c] = __builtin_bit_cast(uint16_t, hv);
      }
      if (c == 0) wsc[rowi] = ldexpf(w[rowi], -e);
    }
    __syncthreads();
  }
}

constexpr int kLsWaves = 4;  // layers per workgroup, one per wave
constexpr int kLsMaxTiles = 64;  // tiles (32 rows) per workgroup at most
constexpr int kLsMaxRows = kLsMaxTiles * 32;

// DC: latent width (128 or 256).  GATHER: rows come from the candidate list.
// CSCALE: a per-row latent scale is given.
//
// The workgroup streams its rows 32 at a time: the global loads of tile it+2
// are issued while tile it is computed, tile it+1 (loaded one step earlier)
// goes to LDS at the end of the step.  Scores collect in LDS (one row per
// layer) and are written in one burst at the end; the level-0 histograms are
// 16-bit, packed two bins per word (a workgroup covers at most 2048 rows).
template <int DC, bool GATHER, bool CSCALE>
__global__ __launch_bounds__(256) void latent_score_kernel(
    const uint16_t* __restrict__ qt16, const float* __restrict__ wsc,
    const uint16_t* __restrict__ latent, const float* __restrict__ c_scale,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ cand, int C, int64_t n_tok,
    int G, int H, int tiles_per_block, int k, float* __restrict__ scores, SelWs sel) {
  constexpr int KSTEPS = DC / 16;  // K = 16 per MFMA
  constexpr int HALF = DC / 2;     // dims per lane half
  constexpr int CPT = DC / 64;     // 8-element chunks per thread per tile
  __shared__ i32x4 lds[2][KSTEPS * 64];
  __shared__ uint32_t lhist[kLsWaves][kSelBins / 2];
  __shared__ __attribute__((aligned(16))) float ssc[kLsWaves][kLsMaxRows];
  __shared__ int32_t sh_n;

  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, g = lane >> 5;
  const int l = blockIdx.z * kLsWaves + wave;
  const bool active = l < G;

  const int64_t off = kv_off[b];
  int64_t n;
  const int32_t* cb = nullptr;
  if constexpr (GATHER) {
    cb = cand + (int64_t)b * C;
    if (threadIdx.x == 0) {
      int lo = 0, hi = C;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cb[mid] < 0) hi = mid; else lo = mid + 1;
      }
      sh_n = lo;
    }
    __syncthreads();
    n = sh_n;
  } else {
    n = kv_off[b + 1] - off;
  }
  const int64_t tok0 = (int64_t)blockIdx.x * tiles_per_block * 32;
  if (tok0 >= n) return;
  int64_t ntl = (n - tok0 + 31) / 32;
  const int ntiles = (int)(ntl < tiles_per_block ? ntl : tiles_per_block);
  const bool select = !GATHER && n > k;
  if constexpr (!GATHER) {
    for (int i = threadIdx.x; i < kLsWaves * kSelBins / 2; i += 256) (&lhist[0][0])[i] = 0;
    // The top-k kernel that follows counts finished segments per (b, l) row.
    if (select && blockIdx.x == 0 && threadIdx.x < kLsWaves && blockIdx.z * kLsWaves + threadIdx.x < G)
      sel.done[(int64_t)b * G + blockIdx.z * kLsWaves + threadIdx.x] = 0u;
  }

  // Absorbed queries (A operand: row = head, K = latent dims; lane half g
  // holds dims HALF*g ..) and the weights of the heads whose results this
  // lane holds (rows 8*(r/4) + 4*g + r%4 of each 32-row block).
  const int la = active ? l : 0;  // inactive waves compute a copy of layer 0 and discard it
  f16x8 qa[2][KSTEPS];
  float wl[2][16];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int row = hb * 32 + col;
    // Clamped, unconditional loads (rows past H are zeroed afterwards).
    const uint16_t* qp = qt16 + (((int64_t)b * G + la) * H + (row < H ? row : H - 1)) * DC + HALF * g;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      i32x4 v = ld16(qp + 8 * j);
      if (row >= H) v = i32x4{0, 0, 0, 0};
      qa[hb][j] = __builtin_bit_cast(f16x8, v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      const float wv = wsc[((int64_t)b * G + la) * H + (head < H ? head : H - 1)];
      wl[hb][r] = head < H ? wv : 0.0f;
    }
  }

  // Producer: thread -> (row pt, dims [p*CPT*8, +CPT*8)).
  const int pt = threadIdx.x & 31, p = threadIdx.x >> 5;
  auto row_of = [&](int64_t s) -> int64_t {
    s = s < n ? s : n - 1;
    if constexpr (GATHER) return off + cb[s];
    else return off + s;
  };
  auto gload = [&](i32x4 (&dst)[CPT], int tile) {
    const int t = tile < ntiles ? tile : ntiles - 1;
    const int64_t r = row_of(tok0 + (int64_t)t * 32 + pt);
    const uint16_t* src = latent + r * DC + p * CPT * 8;
#pragma unroll
    for (int i = 0; i < CPT; ++i) dst[i] = ld16(src + 8 * i);
  };
  auto lstore = [&](int buf, const i32x4 (&src)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int d0 = (p * CPT + i) * 8;
      const int gg = d0 / HALF, jj = (d0 - gg * HALF) / 8;
      lds[buf][jj * 64 + pt + 32 * gg] = bf16x8_to_f16x8(src[i]);
    }
  };
  auto row_scale = [&](int tile) {
    if constexpr (CSCALE) return c_scale[row_of(tok0 + (int64_t)(tile < ntiles ? tile : ntiles - 1) * 32 + col)];
    else return 1.0f;
  };

  auto compute = [&](int buf, int it, float sc) {
    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      const f16x8 kb = __builtin_bit_cast(f16x8, lds[buf][j * 64 + lane]);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[0][j], kb, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[1][j], kb, a1, 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(wl[0][r], relu(a0[r]), part);
      part = fmaf(wl[1][r], relu(a1[r]), part);
    }
    part = sum_halves(part);
    // LDS only from here on; every tile index here is < ntiles.
    const int64_t s = tok0 + (int64_t)it * 32 + col;
    const float val = part * sc;
    if (g == 0) ssc[wave][it * 32 + col] = val;
    if constexpr (!GATHER) {
      const uint32_t bin = score_key(val) >> kSelShift;
      const uint32_t inc = (select && active && g == 0 && s < n) ? 1u : 0u;
      atomicAdd(&lhist[wave][bin >> 1], inc << (16 * (bin & 1)));
    }
  };

  // Ring of two register sets for tiles in flight; the step is unrolled by
  // two so that the set indices are compile-time constants.
  i32x4 pre[2][CPT];
  float skr[2];
  gload(pre[0], 0);
  gload(pre[1], 1);
  skr[0] = row_scale(0);
  skr[1] = row_scale(1);
  lstore(0, pre[0]);
  gload(pre[0], 2);
  __syncthreads();
  const int nsteps = (ntiles + 1) / 2 * 2;
  for (int base = 0; base < nsteps; base += 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int it = base + st;
      if (it < ntiles) {
        compute(st, it, skr[st]);
      }
      skr[st] = row_scale(it + 2);
      lstore(st ^ 1, pre[st ^ 1]);  // tile it+1
      gload(pre[st ^ 1], it + 3);
      __syncthreads();
    }
  }

  // Scores of this workgroup's rows, one burst per layer (16-byte stores
  // where the destination is aligned).
  const int nrow = (int)((n - tok0) < (int64_t)ntiles * 32 ? (n - tok0) : (int64_t)ntiles * 32);
  const int nl = (G - (int)blockIdx.z * kLsWaves) < kLsWaves ? (G - (int)blockIdx.z * kLsWaves) : kLsWaves;
  for (int lw = 0; lw < nl; ++lw) {
    const int lg = blockIdx.z * kLsWaves + lw;
    float* dst = GATHER ? scores + ((int64_t)b * G + lg) * C + tok0 : scores + (int64_t)lg * n_tok + off + tok0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      const int n4 = nrow >> 2;
      for (int i = threadIdx.x; i < n4; i += 256)
        *reinterpret_cast<f32x4*>(dst + 4 * i) = *reinterpret_cast<const f32x4*>(&ssc[lw][4 * i]);
      for (int i = 4 * n4 + threadIdx.x; i < nrow; i += 256) dst[i] = ssc[lw][i];
    } else {
      for (int i = threadIdx.x; i < nrow; i += 256) dst[i] = ssc[lw][i];
    }
  }
  if constexpr (!GATHER) {
    if (!select) return;
    // Each layer's share of its (b, l) row histogram (already 16-bit bins).
    for (int lw = 0; lw < nl; ++lw) {
      const int64_t pi = ((int64_t)b * G + blockIdx.z * kLsWaves + lw) * sel.nwg + blockIdx.x;
      store_partial_packed<256>(lhist[lw], sel.part + pi * kSelBins, sel.cpart + pi * kSelCoarse);
    }
  }
}

}  // namespace

int64_t latent_chunk(int64_t n_tok) {
  int64_t tpb = n_tok / ((int64_t)1024 * 32);
  tpb = tpb < 4 ? 4 : (tpb > kLsMaxTiles ? kLsMaxTiles : tpb);
  return tpb * 32;
}

namespace {

template <bool GATHER, bool CSCALE>
hipError_t launch_ls2(int Dc, dim3 grid, hipStream_t stream, const uint16_t* qt16, const float* wsc,
                      const uint16_t* latent, const float* c_scale, const int64_t* kv_off,
                      const int32_t* cand, int C, int64_t n_tok, int G, int H, int tpb, int k,
                      float* scores, const SelWs& sel) {
  if (Dc == 256)
    latent_score_kernel<256, GATHER, CSCALE><<<grid, dim3(256), 0, stream>>>(
        qt16, wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  else
    latent_score_kernel<128, GATHER, CSCALE><<<grid, dim3(256), 0, stream>>>(
        qt16, wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  return hipGetLastError();
}

template <bool GATHER>
hipError_t launch_ls(int Dc, dim3 grid, hipStream_t stream, const uint16_t* qt16, const float* wsc,
                     const uint16_t* latent, const float* c_scale, const int64_t* kv_off,
                     const int32_t* cand, int C, int64_t n_tok, int G, int H, int tpb, int k,
                     float* scores, const SelWs& sel) {
  if (c_scale)
    return launch_ls2<GATHER, true>(Dc, grid, stream, qt16, wsc, latent, c_scale, kv_off, cand, C, n_tok,
                                    G, H, tpb, k, scores, sel);
  return launch_ls2<GATHER, false>(Dc, grid, stream, qt16, wsc, latent, c_scale, kv_off, cand, C, n_tok, G,
                                   H, tpb, k, scores, sel);
}

}  // namespace

hipError_t launch_latent_absorb(const uint16_t* q, const float* w, const uint16_t* w_dec,
                                int32_t B, int32_t G, int32_t H, int32_t Dh, int32_t Dc,
                                uint16_t* qt16, float* wsc, hipStream_t stream) {
  (void)Dh;
  if (B <= 0) return hipSuccess;
  latent_absorb_kernel<<<dim3((unsigned)(G * H)), dim3(256), 0, stream>>>(q, w, w_dec, B, G, H, Dc,
                                                                          qt16, wsc);
  return hipGetLastError();
}

hipError_t launch_latent_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                               const float* c_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dc,
                               int32_t k, float* scores, const SelWs& sel, hipStream_t stream) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  const int64_t chunk = latent_chunk(n_tok);
  const int64_t tpb = chunk / 32;
  dim3 grid((unsigned)((max_len + chunk - 1) / chunk), (unsigned)B,
            (unsigned)((G + kLsWaves - 1) / kLsWaves));
  return launch_ls<false>(Dc, grid, stream, qt16, wsc, latent, c_scale, kv_off, nullptr, 0, n_tok,
                          G, H, (int)tpb, k, scores, sel);
}

hipError_t launch_hs_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                           const float* c_scale, const int64_t* kv_off, const int32_t* cand,
                           int32_t C, int32_t B, int32_t Gf, int32_t H, int32_t Dc, float* scores,
                           hipStream_t stream) {
  if (B <= 0 || C <= 0) return hipSuccess;
  int64_t tpb = ((int64_t)B * C) / ((int64_t)512 * 32);
  tpb = tpb < 2 ? 2 : (tpb > 32 ? 32 : tpb);
  const int64_t chunk = tpb * 32;
  dim3 grid((unsigned)((C + chunk - 1) / chunk), (unsigned)B,
            (unsigned)((Gf + kLsWaves - 1) / kLsWaves));
  SelWs none = {};
  return launch_ls<true>(Dc, grid, stream, qt16, wsc, latent, c_scale, kv_off, cand, C, 0, Gf, H,
                         (int)tpb, 0, scores, none);
}

}  // namespace li
