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
//   registers and runs v_mfma_f32_16x16x32_f16 against the shared tile, one
//   16-head x 16-row unit at a time, with each unit's ReLU-weighted head
//   reduction on the VALU under the next unit's products.  The gather
//   variant (HS) reads rows kv_off[b] + cand[b][j] instead of contiguous ones.
//   The contiguous variant also builds each (request, layer) row's level-0
//   selection histogram in LDS and stores it as the workgroup's partial.
#include <math.h>

#include "li_device.h"
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kAbsB = 16;  // requests per absorb pass

// bf16 of an fp32 value, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// A positive fp32 block scale split as 2^e * m with m in [1, 2): gfx950's
// scaled fp8 conversion applies only a scale's power of two, so the codes are
// converted exactly times 2^e and the mantissa factor m (rounded to fp16) is
// applied with one packed fp16 multiply.
struct F8Scale {
  float pow2;  // 2^e
  f16x2 m2;    // m, twice
};
__device__ __forceinline__ F8Scale f8_scale(float scale) {
  const uint32_t u = __builtin_bit_cast(uint32_t, scale);
  const _Float16 m = (_Float16)__builtin_bit_cast(float, (u & 0x007FFFFFu) | 0x3F800000u);
  return F8Scale{__builtin_bit_cast(float, u & 0x7F800000u), f16x2{m, m}};
}

// Eight OCP E4M3 values (bytes 8*half .. +7 of v), each times the block
// scale, as fp16: code * 2^e is exact in fp16 (inside its range), then the
// product with m rounds once (nearest even).  One conversion and one packed
// multiply per two values.
__device__ __forceinline__ i32x4 fp8x8_scaled_to_f16x8(i32x4 v, int half, F8Scale sc) {
  const int w[2] = {half ? v[2] : v[0], half ? v[3] : v[1]};
  i32x4 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], sc.pow2, false) * sc.m2;  // bytes 0, 1
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], sc.pow2, true) * sc.m2;   // bytes 2, 3
    r[2 * k] = __builtin_bit_cast(int, lo);
    r[2 * k + 1] = __builtin_bit_cast(int, hi);
  }
  return r;
}

// split = false: qt16[row] = fp16 of the scaled row.  split = true: qt16[row]
// = hi, qt16[nrows + row] = lo, two bf16 parts with hi + lo = the scaled row
// to within 2^-17 of its magnitude (hi is the bf16 rounding, lo that of the
// exact fp32 residual).
//
// One workgroup per (layer l, head h): the [Dc x 128] block of W_l times the
// [128 x B] queries of that head is a small dense contraction, run on bf16
// MFMA (v_mfma_f32_16x16x32_bf16, exact bf16 products, fp32 sums) as 16-row
// tiles of latent dims c against 16 requests, 4 K-steps over the head's 128
// dims.  Wave w holds decoder rows 16 (w nt + i) .. +15 (nt = Dc / 64 tiles)
// in registers for all passes over the batch.  Operand lanes: row or request
// (lane & 15), dims 32 ks + 8 (lane >> 4) .. +7 of K-step ks; the result
// leaves lane (g, n) rows 4 g .. 4 g + 3 of each tile for request n.
__global__ __launch_bounds__(256) void latent_absorb_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ w_dec,
    int B, int G, int H, int Dc, bool split, uint16_t* __restrict__ qt16, float* __restrict__ wsc) {
  constexpr int Dh = 128;
  constexpr int kMaxTiles = 4;  // 16-row tiles per wave at Dc = 256
  __shared__ float red[kAbsB][4];
  const int l = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nt = Dc / 64;
  // All of the wave's decoder loads are issued together, up front (tiles
  // past nt repeat the last one and are never used).
  bf16x8 wa[kMaxTiles][Dh / 32];
#pragma unroll
  for (int i = 0; i < kMaxTiles; ++i) {
    const int c = 16 * (wave * nt + (i < nt ? i : nt - 1)) + col;
    const uint16_t* wrow = w_dec + ((int64_t)l * Dc + c) * (int64_t)H * Dh + (int64_t)h * Dh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < Dh / 32; ++ks) wa[i][ks] = __builtin_bit_cast(bf16x8, ld16(wrow + 32 * ks));
  }

  for (int b0 = 0; b0 < B; b0 += kAbsB) {
    const int nb = (B - b0) < kAbsB ? (B - b0) : kAbsB;
    // Request columns past the batch repeat the last request; their results
    // are never stored.
    const int bq = b0 + (col < nb ? col : nb - 1);
    const uint16_t* qrow = q + (((int64_t)bq * G + l) * H + h) * Dh + 8 * g;
    bf16x8 qb[Dh / 32];
#pragma unroll
    for (int ks = 0; ks < Dh / 32; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, ld16(qrow + 32 * ks));
    f32x4 acc[kMaxTiles];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxTiles; ++i) {
      acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (i < nt) {
#pragma unroll
        for (int ks = 0; ks < Dh / 32; ++ks)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[i][ks], qb[ks], acc[i], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(acc[i][e]));
      }
    }
    // Largest magnitude of request col's absorbed row over all Dc dims: the
    // four lanes of the column, then the four waves.
    am = fmaxf(am, __shfl_xor(am, 16));
    am = fmaxf(am, __shfl_xor(am, 32));
    if (g == 0) red[col][wave] = am;
    __syncthreads();
    const float mx = fmaxf(fmaxf(red[col][0], red[col][1]), fmaxf(red[col][2], red[col][3]));
    int E = 0;
    if (mx > 0.0f) frexpf(mx, &E);
    const int ex = mx > 0.0f ? 15 - E : 0;  // mx * 2^ex in [2^14, 2^15)
    if (col < nb) {
      const int64_t rowi = ((int64_t)(b0 + col) * G + l) * H + h;
#pragma unroll
      for (int i = 0; i < kMaxTiles; ++i) {
        if (i >= nt) continue;
        const int64_t c0 = 16 * (wave * nt + i) + 4 * g;
        uint32_t hv[2], lv[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          uint32_t hp = 0, lp = 0;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const float v = ldexpf(acc[i][2 * e2 + m], ex);
            uint32_t hb, lb = 0;
            if (split) {
              const uint16_t hi = f32_to_bf16_rne(v);
              const float res = v - __builtin_bit_cast(float, (uint32_t)hi << 16);  // exact in fp32
              hb = hi;
              lb = f32_to_bf16_rne(res);
            } else {
              hb = __builtin_bit_cast(uint16_t, (_Float16)v);
            }
            hp |= hb << (16 * m);
            lp |= lb << (16 * m);
          }
          hv[e2] = hp;
          lv[e2] = lp;
        }
        *reinterpret_cast<uint2*>(qt16 + rowi * Dc + c0) = make_uint2(hv[0], hv[1]);
        if (split) *reinterpret_cast<uint2*>(qt16 + ((int64_t)B * G * H + rowi) * Dc + c0) = make_uint2(lv[0], lv[1]);
      }
      if (wave == 0 && g == 0) wsc[rowi] = ldexpf(w[rowi], -ex);
    }
    __syncthreads();  // red is reused by the next pass
  }
}

constexpr int kLsWaves = 4;  // layers per workgroup, one per wave
constexpr int kLsThreads = 64 * kLsWaves;
constexpr int kLsMaxTiles = 64;  // tiles (32 rows) per workgroup at most
constexpr int kLsMaxRows = kLsMaxTiles * 32;

// DC: latent width (128, 192 or 256).  GATHER: rows come from the candidate list.
// CSCALE: a per-row latent scale is given.
//
// Wave l holds its layer's 64 x DC absorbed query in registers (four 16-head
// blocks).  A 32-row tile is eight units (16-row block rb x head block hb),
// each a chain of DC/32 v_mfma_f32_16x16x32_f16 products over all the dims;
// the epilogue of unit n (ReLU and head weights, on the VALU) runs while the
// products of unit n + 1 execute, and the tile producer's conversion runs
// between the two row blocks.  A lane's unit results are 4 heads of one row;
// after the tile a permlane32 and a permlane16 swap fold the four lane
// groups' sums, leaving row block 0 in lanes 0-15 and row block 1 in lanes
// 32-47.  The workgroup stages 32 latent rows at a time through LDS,
// converted bf16 -> fp16 once and shared by its four waves; two workgroups
// fit on a CU, so each SIMD runs waves of two workgroups that pass their
// barriers at different times.  Scores collect in LDS and are written in one
// burst at the end; the level-0 histograms are 16-bit, packed two bins per
// word (a workgroup covers at most 2048 rows).
template <int DC, bool GATHER, bool CSCALE, bool F8>
__global__ __launch_bounds__(kLsThreads, 2) void latent_score_kernel(
    const uint16_t* __restrict__ qt16, const float* __restrict__ wsc,
    const uint16_t* __restrict__ latent, const float* __restrict__ c_scale,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ cand, int C, int64_t n_tok,
    int G, int H, int tiles_per_block, int k, float* __restrict__ scores, SelWs sel) {
  constexpr int KS = DC / 32;   // products per unit (K = 32 each)
  constexpr int NCR = DC / 8;   // 16-byte chunks per latent row
  constexpr int CPT = NCR / 8;  // chunks per producer thread (8 threads per row)
  constexpr int NBLK = (DC + 127) / 128;  // fp8 block scales per row
  // fp8 rows whose width is not a multiple of 128 (Dc = 192): a thread's 8*CPT
  // values can straddle a block boundary and need not be 16-byte aligned, so
  // they come as 8-byte chunks, each with its own block's scale.
  constexpr bool F8N = F8 && (DC % 128 != 0);
  static_assert(CPT >= 1 && CPT * 8 == NCR && 32 * 8 == kLsThreads, "tile producer layout");
  // Tile slot in MFMA fragment order: the 16 bytes lane l needs for product s
  // of row block rb sit at (rb * KS + s) * 64 + l, so fragment reads are
  // lane-linear; producer lanes (one row each) also write consecutive slots.
  __shared__ i32x4 ktile[2][32 * NCR];
  __shared__ uint32_t lhist[kLsWaves][kSelBins / 2];
  __shared__ __attribute__((aligned(16))) float ssc[kLsWaves][kLsMaxRows];
  __shared__ int32_t sh_n;

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int c16 = lane & 15, g4 = lane >> 4;
  const int l = blockIdx.z * kLsWaves + wave;
  const bool active = l < G;

  const int64_t off = kv_off[b];
  int64_t n;
  const int32_t* cb = nullptr;
  if constexpr (GATHER) {
    // Valid candidates come first, then -1 padding.  This workgroup only
    // reads its own range tok0 .. tok0 + 32 * tiles_per_block - 1, so the
    // valid ones there, counted from one round of loads, give n for it
    // (tok0 + that count; every use of n below is inside the range).
    cb = cand + (int64_t)b * C;
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_block * 32;
    if (tid == 0) sh_n = 0;
    __syncthreads();
    uint32_t cv = 0;
    for (int i = tid; i < tiles_per_block * 32; i += kLsThreads)
      cv += (t0 + i < C && cb[t0 + i] >= 0) ? 1u : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cv += (uint32_t)__shfl_xor((int)cv, o);
    if ((tid & 63) == 0) atomicAdd(&sh_n, (int32_t)cv);
    __syncthreads();
    n = t0 + sh_n;
  } else {
    n = kv_off[b + 1] - off;
  }
  const int64_t tok0 = (int64_t)blockIdx.x * tiles_per_block * 32;
  if (tok0 >= n) return;
  const int64_t ntl = (n - tok0 + 31) / 32;
  const int ntiles = (int)(ntl < tiles_per_block ? ntl : tiles_per_block);
  const bool select = !GATHER && n > k;
  if constexpr (!GATHER) {
    for (int i = tid; i < kLsWaves * kSelBins / 2; i += kLsThreads) (&lhist[0][0])[i] = 0;
    // The top-k kernel that follows counts finished segments per (b, l) row.
    if (select && blockIdx.x == 0 && tid < kLsWaves && blockIdx.z * kLsWaves + tid < G)
      sel.done[(int64_t)b * G + blockIdx.z * kLsWaves + tid] = 0u;
  }

  // Absorbed query as the A operand (row = head 16*hb + c16, dims 32*s +
  // 8*g4 .. +7 of product s) and the weights of the heads whose results this
  // lane holds (rows 4*g4 + r of each block).
  const int la = active ? l : 0;
  f16x8 qa[4][KS];
  float wl[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = 16 * hb + c16;
    // Clamped, unconditional loads (rows past H are zeroed afterwards).
    const uint16_t* qp = qt16 + (((int64_t)b * G + la) * H + (head < H ? head : H - 1)) * DC + 8 * g4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      i32x4 v = ld16(qp + 32 * s);
      if (head >= H) v = i32x4{0, 0, 0, 0};
      qa[hb][s] = __builtin_bit_cast(f16x8, v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 16 * hb + 4 * g4 + r;
      const float wv = wsc[((int64_t)b * G + la) * H + (hr < H ? hr : H - 1)];
      wl[hb][r] = hr < H ? wv : 0.0f;
    }
  }

  // Producer: thread -> row pt of the tile, chunks CPT*p .. +CPT-1.
  const int pt = tid & 31, p = tid >> 5;
  auto row_of = [&](int64_t s) -> int64_t {
    s = s < n ? s : n - 1;
    if constexpr (GATHER) return off + cb[s];
    else return off + s;
  };
  // F8: the thread's 8*CPT values are 8*CPT fp8 bytes (CPT / 2 loads) inside
  // one 128-value block, whose scale comes with them; F8N: CPT 8-byte loads
  // (chunk i in dst[i].xy) and the scales of the blocks they fall in.
  // The gather's candidate index of the producer's row in a tile, loaded one
  // step ahead of that tile's latent row so the two loads do not chain.
  auto cidx_of = [&](int tile) -> int64_t {
    if constexpr (GATHER) {
      int64_t s = tok0 + (int64_t)(tile < ntiles ? tile : ntiles - 1) * 32 + pt;
      return cb[s < n ? s : n - 1];
    } else {
      return 0;
    }
  };
  auto gload_row = [&](i32x4 (&dst)[CPT], float (&bsc)[2], int64_t row) {
    if constexpr (F8N) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(latent) + row * DC + 8 * CPT * p;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const i32x2 v = *reinterpret_cast<const i32x2*>(src + 8 * i);
        dst[i] = i32x4{v.x, v.y, 0, 0};
      }
      const int b0 = 8 * CPT * p / 128, b1 = (8 * CPT * p + 8 * CPT - 1) / 128;
      bsc[0] = c_scale[row * NBLK + b0];
      bsc[1] = c_scale[row * NBLK + b1];
    } else if constexpr (F8) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(latent) + row * DC + 8 * CPT * p;
#pragma unroll
      for (int i = 0; i < CPT / 2; ++i) dst[i] = ld16(src + 16 * i);
      bsc[0] = bsc[1] = c_scale[row * NBLK + 8 * CPT * p / 128];
    } else {
      const uint16_t* src = latent + row * DC + 8 * CPT * p;
#pragma unroll
      for (int i = 0; i < CPT; ++i) dst[i] = ld16(src + 8 * i);
      bsc[0] = bsc[1] = 1.0f;
    }
  };
  auto gload = [&](i32x4 (&dst)[CPT], float (&bsc)[2], int tile) {
    const int t = tile < ntiles ? tile : ntiles - 1;
    gload_row(dst, bsc, row_of(tok0 + (int64_t)t * 32 + pt));
  };
  auto lstore = [&](int slot, const i32x4 (&src)[CPT], const float (&bsc)[2]) {
    F8Scale f0 = {}, f1 = {};
    if constexpr (F8) f0 = f8_scale(bsc[0]);
    if constexpr (F8N) f1 = f8_scale(bsc[1]);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = CPT * p + i;
      i32x4 v;
      if constexpr (F8N) {
        // chunk c holds values 8c .. 8c+7, all in block 8c / 128
        const bool second = (8 * c) / 128 != (8 * CPT * p) / 128;
        v = fp8x8_scaled_to_f16x8(src[i], 0, second ? f1 : f0);
      } else if constexpr (F8) {
        v = fp8x8_scaled_to_f16x8(src[i >> 1], i & 1, f0);
      } else {
        v = bf16x8_to_f16x8(src[i]);
      }
      ktile[slot][((pt >> 4) * KS + (c >> 2)) * 64 + (c & 3) * 16 + (pt & 15)] = v;
    }
  };
  // B operand of row block rb, product s: row 16*rb + c16, dims 32*s + 8*g4 .. +7.
  auto bfrag = [&](int slot, int rb, i32x4 (&dst)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s] = ktile[slot][(rb * KS + s) * 64 + lane];
  };
  // This lane's row after the fold: row block lane >> 5, row c16 of it.
  const int frow = 16 * (lane >> 5) + c16;
  auto row_scale = [&](int tile) {
    if constexpr (CSCALE) return c_scale[row_of(tok0 + (int64_t)(tile < ntiles ? tile : ntiles - 1) * 32 + frow)];
    else return 1.0f;
  };

  // Step i computes tile i from LDS slot i & 1, writes tile i+1 into the
  // other slot (whose readers finished tile i-1 before the previous barrier)
  // and loads tile i+3 into the register set tile i+1 had.
  i32x4 gk[2][CPT];
  float gs[2][2];
  float skr[2];
  gload(gk[0], gs[0], 0);
  gload(gk[1], gs[1], 1);
  skr[0] = row_scale(0);
  lstore(0, gk[0], gs[0]);
  gload(gk[0], gs[0], 2);
  int64_t cnext = cidx_of(3);  // gather: the index of the producer's row of tile 3
  __syncthreads();
  const int nsteps = (ntiles + 1) / 2 * 2;
  for (int base = 0; base < nsteps; base += 2) {
    set_progress_priority(base, nsteps);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int it = base + st;
      const bool work = active && it < ntiles;  // uniform across the wave
      skr[st ^ 1] = row_scale(it + 1);
      i32x4 bk[KS];
      f32x4 acc[8];
      float P0 = 0.0f, P1 = 0.0f;
      auto issue = [&](int u) {  // unit u: row block u >> 2 (in bk), head block u & 3
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          a = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[u & 3][s], __builtin_bit_cast(f16x8, bk[s]), a, 0, 0, 0);
        acc[u] = a;
      };
      auto epi = [&](int u) {
        float& P = (u >> 2) ? P1 : P0;
#pragma unroll
        for (int r = 0; r < 4; ++r) P = fmaf(wl[u & 3][r], relu(acc[u][r]), P);
      };
      if (work) {
        bfrag(st, 0, bk);
        issue(0);
        issue(1);
        __builtin_amdgcn_sched_barrier(0);
        epi(0);
        __builtin_amdgcn_sched_barrier(0);
        issue(2);
        __builtin_amdgcn_sched_barrier(0);
        epi(1);
        __builtin_amdgcn_sched_barrier(0);
        issue(3);
        __builtin_amdgcn_sched_barrier(0);
        epi(2);
        __builtin_amdgcn_sched_barrier(0);
        bfrag(st, 1, bk);
      }
      lstore(st ^ 1, gk[st ^ 1], gs[st ^ 1]);
      if constexpr (GATHER) {
        gload_row(gk[st ^ 1], gs[st ^ 1], off + cnext);
        cnext = cidx_of(it + 4);
      } else {
        gload(gk[st ^ 1], gs[st ^ 1], it + 3);
      }
      if (work) {
        __builtin_amdgcn_sched_barrier(0);
        issue(4);
        __builtin_amdgcn_sched_barrier(0);
        epi(3);
        __builtin_amdgcn_sched_barrier(0);
        issue(5);
        __builtin_amdgcn_sched_barrier(0);
        epi(4);
        __builtin_amdgcn_sched_barrier(0);
        issue(6);
        __builtin_amdgcn_sched_barrier(0);
        epi(5);
        __builtin_amdgcn_sched_barrier(0);
        issue(7);
        __builtin_amdgcn_sched_barrier(0);
        epi(6);
        epi(7);
        const float R = swap_sum32(P0, P1);
        const float val = swap_sum16(R, R) * skr[st];
        if ((g4 & 1) == 0) {
          ssc[wave][it * 32 + frow] = val;
          if constexpr (!GATHER) {
            const uint32_t bin = score_key(val) >> kSelShift;
            const uint32_t inc = (select && tok0 + it * 32 + frow < n) ? 1u : 0u;
            atomicAdd(&lhist[wave][bin >> 1], inc << (16 * (bin & 1)));
          }
        }
      }
      __syncthreads();
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // Scores of this workgroup's rows, one burst per layer (16-byte stores
  // where the destination is aligned).
  const int nrow = (int)((n - tok0) < (int64_t)ntiles * 32 ? (n - tok0) : (int64_t)ntiles * 32);
  const int nl = (G - (int)blockIdx.z * kLsWaves) < kLsWaves ? (G - (int)blockIdx.z * kLsWaves) : kLsWaves;
  for (int lw = 0; lw < nl; ++lw) {
    const int lg = blockIdx.z * kLsWaves + lw;
    float* dst = GATHER ? scores + ((int64_t)b * G + lg) * C + tok0 : scores + (int64_t)lg * n_tok + off + tok0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      const int n4 = nrow >> 2;
      for (int i = tid; i < n4; i += kLsThreads)
        *reinterpret_cast<f32x4*>(dst + 4 * i) = *reinterpret_cast<const f32x4*>(&ssc[lw][4 * i]);
      for (int i = 4 * n4 + tid; i < nrow; i += kLsThreads) dst[i] = ssc[lw][i];
    } else {
      for (int i = tid; i < nrow; i += kLsThreads) dst[i] = ssc[lw][i];
    }
  }
  if constexpr (!GATHER) {
    if (!select) return;
    // Each layer's share of its (b, l) row histogram (already 16-bit bins).
    for (int lw = 0; lw < nl; ++lw) {
      const int64_t pi = ((int64_t)b * G + blockIdx.z * kLsWaves + lw) * sel.nwg + blockIdx.x;
      store_partial_packed<kLsThreads>(lhist[lw], sel.part + pi * kSelBins, sel.cpart + pi * kSelCoarse);
    }
  }
}

constexpr int kSpWaves = 8;               // LI_LATENT_SPLIT_BF16 scan: one wave per (layer, head half)
constexpr int kSpLayers = kSpWaves / 2;   // layers per workgroup
constexpr int kSpThreads = 64 * kSpWaves;

// The LI_LATENT_SPLIT_BF16 form of the scan: the absorbed query is hi + lo
// (two bf16 rows) and the latent is used as stored (bf16), so each product
// is two v_mfma_f32_16x16x32_bf16 into one accumulator.  The query of 64
// heads would take all 256 registers of a wave in this form, so a wave holds
// half the heads of one layer (two 16-head blocks, hi and lo: 128 VGPRs at
// Dc = 256) and the two halves of a layer meet in an LDS float add of their
// scaled partial sums (two partials added to zero give the same bits in
// either order).  A 32-row tile is four units (16-row block x head block),
// each unit's epilogue running under the next unit's products; the latent
// tile goes through LDS once, unconverted, in MFMA-fragment order.  After the
// last tile one pass writes the scores out and builds the level-0
// histograms of the contiguous variant.
template <int DC, bool GATHER, bool CSCALE>
__global__ __launch_bounds__(kSpThreads) void latent_split_kernel(
    const uint16_t* __restrict__ qhi, const uint16_t* __restrict__ qlo, const float* __restrict__ wsc,
    const uint16_t* __restrict__ latent, const float* __restrict__ c_scale,
    const int64_t* __restrict__ kv_off, const int32_t* __restrict__ cand, int C, int64_t n_tok,
    int G, int H, int tiles_per_block, int k, float* __restrict__ scores, SelWs sel) {
  constexpr int KS = DC / 32;    // products per unit and query part (K = 32 each)
  constexpr int NCR = DC / 8;    // 16-byte chunks per latent row
  constexpr int CPT = (NCR + 15) / 16;  // chunks per producer thread (up to 16 threads per row)
  constexpr int NPROD = NCR / CPT;      // producer threads per row (12 at Dc = 192, else 16)
  static_assert(CPT * NPROD == NCR && 32 * 16 == kSpThreads && NPROD % 2 == 0, "tile producer layout");
  // Tile slot in MFMA fragment order: the 16 bytes lane l needs for product s
  // of row block rb sit at (rb * KS + s) * 64 + l.
  __shared__ i32x4 ktile[2][32 * NCR];
  __shared__ uint32_t lhist[kSpLayers][kSelBins / 2];
  __shared__ __attribute__((aligned(16))) float ssc[kSpLayers][kLsMaxRows];
  __shared__ int32_t sh_n;

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int c16 = lane & 15, g4 = lane >> 4;
  const int lw = wave >> 1, hh = wave & 1;
  const int l = blockIdx.z * kSpLayers + lw;
  const bool active = l < G;

  const int64_t off = kv_off[b];
  int64_t n;
  const int32_t* cb = nullptr;
  if constexpr (GATHER) {
    // Valid candidates come first, then -1 padding.  This workgroup only
    // reads its own range tok0 .. tok0 + 32 * tiles_per_block - 1, so the
    // valid ones there, counted from one round of loads, give n for it
    // (tok0 + that count; every use of n below is inside the range).
    cb = cand + (int64_t)b * C;
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_block * 32;
    if (tid == 0) sh_n = 0;
    __syncthreads();
    uint32_t cv = 0;
    for (int i = tid; i < tiles_per_block * 32; i += kSpThreads)
      cv += (t0 + i < C && cb[t0 + i] >= 0) ? 1u : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cv += (uint32_t)__shfl_xor((int)cv, o);
    if ((tid & 63) == 0) atomicAdd(&sh_n, (int32_t)cv);
    __syncthreads();
    n = t0 + sh_n;
  } else {
    n = kv_off[b + 1] - off;
  }
  const int64_t tok0 = (int64_t)blockIdx.x * tiles_per_block * 32;
  if (tok0 >= n) return;
  const int64_t ntl = (n - tok0 + 31) / 32;
  const int ntiles = (int)(ntl < tiles_per_block ? ntl : tiles_per_block);
  const bool select = !GATHER && n > k;
  for (int i = tid; i < kSpLayers * kSelBins / 2; i += kSpThreads) (&lhist[0][0])[i] = 0;
  for (int i = tid; i < kSpLayers * kLsMaxRows / 4; i += kSpThreads)
    reinterpret_cast<f32x4*>(&ssc[0][0])[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (!GATHER) {
    // The top-k kernel that follows counts finished segments per (b, l) row.
    if (select && blockIdx.x == 0 && tid < kSpLayers && blockIdx.z * kSpLayers + tid < G)
      sel.done[(int64_t)b * G + blockIdx.z * kSpLayers + tid] = 0u;
  }

  // Query parts as A operands (row = head 32*hh + 16*hb + c16, dims 32*s +
  // 8*g4 .. +7 of product s) and the weights of the heads whose results this
  // lane holds (rows 4*g4 + r of each block).
  const int la = active ? l : 0;
  bf16x8 qh[2][KS], ql[2][KS];
  float wl[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * hh + 16 * hb + c16;
    // Clamped, unconditional loads (rows past H are zeroed afterwards).
    const int64_t qo = (((int64_t)b * G + la) * H + (head < H ? head : H - 1)) * DC + 8 * g4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      i32x4 vh = ld16(qhi + qo + 32 * s), vl = ld16(qlo + qo + 32 * s);
      if (head >= H) vh = vl = i32x4{0, 0, 0, 0};
      qh[hb][s] = __builtin_bit_cast(bf16x8, vh);
      ql[hb][s] = __builtin_bit_cast(bf16x8, vl);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hr = 32 * hh + 16 * hb + 4 * g4 + r;
      const float wv = wsc[((int64_t)b * G + la) * H + (hr < H ? hr : H - 1)];
      wl[hb][r] = hr < H ? wv : 0.0f;
    }
  }

  // Producer: thread -> row pt of the tile, chunks CPT*p .. +CPT-1.
  const int pt = tid & 31, p = tid >> 5;
  auto row_of = [&](int64_t s) -> int64_t {
    s = s < n ? s : n - 1;
    if constexpr (GATHER) return off + cb[s];
    else return off + s;
  };
  // Threads p >= NPROD (a pair of whole waves at Dc = 192) load a valid chunk
  // too, so the loads stay unconditional, and store nothing.
  const int pp = p < NPROD ? p : NPROD - 1;
  auto gload = [&](i32x4 (&dst)[CPT], int tile) {
    const int t = tile < ntiles ? tile : ntiles - 1;
    const uint16_t* src = latent + row_of(tok0 + (int64_t)t * 32 + pt) * DC + 8 * CPT * pp;
#pragma unroll
    for (int i = 0; i < CPT; ++i) dst[i] = ld16(src + 8 * i);
  };
  auto lstore = [&](int slot, const i32x4 (&src)[CPT]) {
    if (NPROD * 32 < kSpThreads && p >= NPROD) return;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = CPT * p + i;
      ktile[slot][((pt >> 4) * KS + (c >> 2)) * 64 + (c & 3) * 16 + (pt & 15)] = src[i];
    }
  };
  auto bfrag = [&](int slot, int rb, i32x4 (&dst)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s] = ktile[slot][(rb * KS + s) * 64 + lane];
  };
  // This lane's row after the fold: row block lane >> 5, row c16 of it.
  const int frow = 16 * (lane >> 5) + c16;
  auto row_scale = [&](int tile) {
    if constexpr (CSCALE) return c_scale[row_of(tok0 + (int64_t)(tile < ntiles ? tile : ntiles - 1) * 32 + frow)];
    else return 1.0f;
  };

  // Step i computes tile i from LDS slot i & 1, writes tile i+1 into the
  // other slot (whose readers finished tile i-1 before the previous barrier)
  // and loads tile i+3 into the register set tile i+1 had.
  i32x4 gk[2][CPT];
  float skr[2];
  gload(gk[0], 0);
  gload(gk[1], 1);
  skr[0] = row_scale(0);
  lstore(0, gk[0]);
  gload(gk[0], 2);
  __syncthreads();
  const int nsteps = (ntiles + 1) / 2 * 2;
  for (int base = 0; base < nsteps; base += 2) {
    set_progress_priority(base, nsteps);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int it = base + st;
      const bool work = active && it < ntiles;  // uniform across the wave
      skr[st ^ 1] = row_scale(it + 1);
      i32x4 bk[KS];
      f32x4 acc[4];
      float P0 = 0.0f, P1 = 0.0f;
      auto issue = [&](int u) {  // unit u: row block u >> 1 (in bk), head block u & 1
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kb = __builtin_bit_cast(bf16x8, bk[s]);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[u & 1][s], kb, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[u & 1][s], kb, a, 0, 0, 0);
        }
        acc[u] = a;
      };
      auto epi = [&](int u) {
        float& P = (u >> 1) ? P1 : P0;
#pragma unroll
        for (int r = 0; r < 4; ++r) P = fmaf(wl[u & 1][r], relu(acc[u][r]), P);
      };
      if (work) {
        bfrag(st, 0, bk);
        issue(0);
        issue(1);
        __builtin_amdgcn_sched_barrier(0);
        epi(0);
        __builtin_amdgcn_sched_barrier(0);
        bfrag(st, 1, bk);
      }
      lstore(st ^ 1, gk[st ^ 1]);
      gload(gk[st ^ 1], it + 3);
      if (work) {
        __builtin_amdgcn_sched_barrier(0);
        issue(2);
        __builtin_amdgcn_sched_barrier(0);
        epi(1);
        __builtin_amdgcn_sched_barrier(0);
        issue(3);
        __builtin_amdgcn_sched_barrier(0);
        epi(2);
        epi(3);
        const float R = swap_sum32(P0, P1);
        const float part = swap_sum16(R, R) * skr[st];
        if ((g4 & 1) == 0) atomicAdd(&ssc[lw][it * 32 + frow], part);
      }
      __syncthreads();
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // Scores of this workgroup's rows, one pass per layer (16-byte stores where
  // the destination is aligned), and their histogram counts.
  const int nrow = (int)((n - tok0) < (int64_t)ntiles * 32 ? (n - tok0) : (int64_t)ntiles * 32);
  const int nl = (G - (int)blockIdx.z * kSpLayers) < kSpLayers ? (G - (int)blockIdx.z * kSpLayers) : kSpLayers;
  auto count = [&](int ly, float v) {
    const uint32_t bin = score_key(v) >> kSelShift;
    atomicAdd(&lhist[ly][bin >> 1], 1u << (16 * (bin & 1)));
  };
  for (int ly = 0; ly < nl; ++ly) {
    const int lg = blockIdx.z * kSpLayers + ly;
    float* dst = GATHER ? scores + ((int64_t)b * G + lg) * C + tok0 : scores + (int64_t)lg * n_tok + off + tok0;
    int done = 0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      const int n4 = nrow >> 2;
      for (int i = tid; i < n4; i += kSpThreads) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&ssc[ly][4 * i]);
        *reinterpret_cast<f32x4*>(dst + 4 * i) = v;
        if (select) {
          count(ly, v[0]);
          count(ly, v[1]);
          count(ly, v[2]);
          count(ly, v[3]);
        }
      }
      done = 4 * n4;
    }
    for (int i = done + tid; i < nrow; i += kSpThreads) {
      const float v = ssc[ly][i];
      dst[i] = v;
      if (select) count(ly, v);
    }
  }
  if constexpr (!GATHER) {
    if (!select) return;
    __syncthreads();
    // Each layer's share of its (b, l) row histogram (already 16-bit bins).
    for (int ly = 0; ly < nl; ++ly) {
      const int64_t pi = ((int64_t)b * G + blockIdx.z * kSpLayers + ly) * sel.nwg + blockIdx.x;
      store_partial_packed<kSpThreads>(lhist[ly], sel.part + pi * kSelBins, sel.cpart + pi * kSelCoarse);
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

// qlo: the lo parts of the split form (ignored otherwise).
template <bool GATHER, bool CSCALE>
hipError_t launch_ls2(bool split, int Dc, dim3 grid, hipStream_t stream, const uint16_t* qt16,
                      const uint16_t* qlo, const float* wsc, const uint16_t* latent, const float* c_scale,
                      const int64_t* kv_off, const int32_t* cand, int C, int64_t n_tok, int G, int H, int tpb,
                      int k, float* scores, const SelWs& sel) {
  static_assert(kSpLayers == kLsWaves, "both forms cover the same layers per workgroup (grid z)");
  if (split) {
    if (Dc == 256)
      return launch_kernel(latent_split_kernel<256, GATHER, CSCALE>, grid, dim3(kSpThreads), 0, stream, qt16, qlo,
                           wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
    if (Dc == 192)
      return launch_kernel(latent_split_kernel<192, GATHER, CSCALE>, grid, dim3(kSpThreads), 0, stream, qt16, qlo,
                           wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
    return launch_kernel(latent_split_kernel<128, GATHER, CSCALE>, grid, dim3(kSpThreads), 0, stream, qt16, qlo,
                         wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  }
  if (Dc == 256)
    return launch_kernel(latent_score_kernel<256, GATHER, CSCALE, false>, grid, dim3(kLsThreads), 0, stream, qt16,
                         wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  if (Dc == 192)
    return launch_kernel(latent_score_kernel<192, GATHER, CSCALE, false>, grid, dim3(kLsThreads), 0, stream, qt16,
                         wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  return launch_kernel(latent_score_kernel<128, GATHER, CSCALE, false>, grid, dim3(kLsThreads), 0, stream, qt16,
                       wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
}

// fp8 latent (c_scale = its block scales, required): the fp16 form only.
template <bool GATHER>
hipError_t launch_ls8(int Dc, dim3 grid, hipStream_t stream, const uint16_t* qt16, const float* wsc,
                      const uint16_t* latent, const float* c_scale, const int64_t* kv_off, const int32_t* cand, int C,
                      int64_t n_tok, int G, int H, int tpb, int k, float* scores, const SelWs& sel) {
  if (Dc == 256)
    return launch_kernel(latent_score_kernel<256, GATHER, false, true>, grid, dim3(kLsThreads), 0, stream, qt16,
                         wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  if (Dc == 192)
    return launch_kernel(latent_score_kernel<192, GATHER, false, true>, grid, dim3(kLsThreads), 0, stream, qt16,
                         wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
  return launch_kernel(latent_score_kernel<128, GATHER, false, true>, grid, dim3(kLsThreads), 0, stream, qt16,
                       wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k, scores, sel);
}

template <bool GATHER>
hipError_t launch_ls(bool split, bool fp8, int Dc, dim3 grid, hipStream_t stream, const uint16_t* qt16,
                     const uint16_t* qlo, const float* wsc, const uint16_t* latent, const float* c_scale,
                     const int64_t* kv_off, const int32_t* cand, int C, int64_t n_tok, int G, int H, int tpb,
                     int k, float* scores, const SelWs& sel) {
  if (fp8)
    return launch_ls8<GATHER>(Dc, grid, stream, qt16, wsc, latent, c_scale, kv_off, cand, C, n_tok, G, H, tpb, k,
                              scores, sel);
  if (c_scale)
    return launch_ls2<GATHER, true>(split, Dc, grid, stream, qt16, qlo, wsc, latent, c_scale, kv_off, cand, C,
                                    n_tok, G, H, tpb, k, scores, sel);
  return launch_ls2<GATHER, false>(split, Dc, grid, stream, qt16, qlo, wsc, latent, c_scale, kv_off, cand, C,
                                   n_tok, G, H, tpb, k, scores, sel);
}

}  // namespace

hipError_t launch_latent_absorb(const uint16_t* q, const float* w, const uint16_t* w_dec,
                                int32_t B, int32_t G, int32_t H, int32_t Dh, int32_t Dc, bool split,
                                uint16_t* qt16, float* wsc, hipStream_t stream) {
  (void)Dh;
  if (B <= 0) return hipSuccess;
  return launch_kernel(latent_absorb_kernel, dim3((unsigned)(G * H)), dim3(256), 0, stream, q, w, w_dec, B, G, H, Dc,
                       split, qt16, wsc);
}

hipError_t launch_latent_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                               const float* c_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dc,
                               int32_t k, bool split, bool fp8, float* scores, const SelWs& sel,
                               hipStream_t stream) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  const int64_t chunk = latent_chunk(n_tok);
  const int64_t tpb = chunk / 32;
  dim3 grid((unsigned)((max_len + chunk - 1) / chunk), (unsigned)B,
            (unsigned)((G + kLsWaves - 1) / kLsWaves));
  const uint16_t* qlo = qt16 + (int64_t)B * G * H * Dc;
  return launch_ls<false>(split, fp8, Dc, grid, stream, qt16, qlo, wsc, latent, c_scale, kv_off, nullptr, 0,
                          n_tok, G, H, (int)tpb, k, scores, sel);
}

hipError_t launch_hs_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                           const float* c_scale, const int64_t* kv_off, const int32_t* cand,
                           int32_t C, int32_t B, int32_t Gf, int32_t H, int32_t Dc, bool split, bool fp8,
                           float* scores, hipStream_t stream) {
  if (B <= 0 || C <= 0) return hipSuccess;
  int64_t tpb = ((int64_t)B * C) / ((int64_t)512 * 32);
  tpb = tpb < 2 ? 2 : (tpb > 32 ? 32 : tpb);
  const int64_t chunk = tpb * 32;
  dim3 grid((unsigned)((C + chunk - 1) / chunk), (unsigned)B,
            (unsigned)((Gf + kLsWaves - 1) / kLsWaves));
  SelWs none = {};
  const uint16_t* qlo = qt16 + (int64_t)B * Gf * H * Dc;
  return launch_ls<true>(split, fp8, Dc, grid, stream, qt16, qlo, wsc, latent, c_scale, kv_off, cand, C, 0, Gf,
                         H, (int)tpb, 0, scores, none);
}

}  // namespace li
