// Latent-cache append: the group's shared latent row of each new token,
// c = W_enc h, computed from the first layer's hidden state and written into
// the latent cache at the token's row.
//
// Source: "LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for
// Sparse Attention", Abstract and Figure 1 (one latent cache per layer group,
// derived from the group's first-layer hidden states).  The encoder's form is
// not on the page; it is read as a linear down-projection, the latent of
// Multi-head Latent Attention that the page extends.
//
// The product is a dense contraction [M][d_model] x [d_model][Dc] with a
// small Dc (128, 192 or 256) and a long K, so it runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  A workgroup takes 128 hidden-state rows and
// every latent column, so h is read from HBM once; K is split over `S`
// workgroups so that a few thousand rows still fill the chip.  With S > 1
// each split writes an fp32 partial tile and a second kernel sums the splits
// in a fixed order, rounds to bf16 (nearest, ties to even) and scatters the
// rows to dst_row: the result does not depend on the order workgroups run in.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kApRows = 128;  // hidden-state rows per workgroup
constexpr int kApK = 64;      // K elements per pipeline step (two MFMA K blocks)
constexpr int kApWaves = 8;
constexpr int kApThreads = 64 * kApWaves;
constexpr int kApSlotsA = kApRows / 16 * 2 * 64;  // 16-byte fragment slots of the h tile
#ifndef LI_APPEND_DEPTH
#define LI_APPEND_DEPTH 2
#endif
constexpr int kApDepth = LI_APPEND_DEPTH;  // K steps loaded ahead of their use

// Lanes per row in the split sum: Dc / 4 quads rounded up to a power of two.
__host__ __device__ constexpr int append_row_lanes(int dc) { return dc / 4 <= 32 ? 32 : (dc / 4 <= 64 ? 64 : 128); }

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// OCP E4M3FN code of a finite fp32 value: nearest, ties to even, saturated at
// 448 (the codes past it are NaN).  Normal range: the fp32 mantissa rounded to
// 3 bits (a carry moves into the exponent), exponent rebiased 127 -> 7; below
// 2^-6 the spacing is 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 464.f) {
    code = 0x7Eu;  // 464 is the tie between 448 and 480: 448 is the even one
  } else if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);  // 8 gives 0x08, the smallest normal
  } else {
    const uint32_t au = u & 0x7FFFFFFFu;
    code = ((au + 0x7FFFFu + ((au >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sgn | code;
}

// LDS holds each K step's tiles in MFMA fragment order: slot
// ((t * 2 + ks) * 64 + lane) is the 16 bytes that `lane` feeds to the MFMA of
// 16-row tile t and K block ks: row t*16 + (lane & 15), K elements
// 16*(lane >> 4) + 8*ks .. +7 of the step's 64.  The MFMA sums over its 32 K
// positions, so any assignment of the step's K elements to (ks, lane group)
// is the same product as long as both operands use it; this one gives each
// producer thread 32 contiguous bytes (its two ks slots), so four lanes read
// a whole 128-byte line of a row.  Fragment reads and LDS writes are
// consecutive per wave.
template <int DC, int D>
__global__ __launch_bounds__(kApThreads, 1) void append_gemm_kernel(
    const uint16_t* h, const uint16_t* w_enc, const int64_t* __restrict__ dst,
    int32_t M, int32_t d_model, int32_t steps_per_split, float* __restrict__ part,
    uint16_t* __restrict__ latent) {
  constexpr int kSlotsB = DC / 16 * 2 * 64;
  constexpr int kPerA = kApSlotsA / 2 / kApThreads;  // 32-byte slot pairs per thread
  constexpr int kPairsB = kSlotsB / 2;
  constexpr int kPerB = (kPairsB + kApThreads - 1) / kApThreads;  // the last pass partial at Dc = 192
  constexpr int kWct = DC / 16 / 4;  // 16-column tiles per wave
  static_assert(2 * kPerA * kApThreads == kApSlotsA && kWct * 64 == DC, "tile split");
  __shared__ i32x4 tile[2][kApSlotsA + kSlotsB];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wr = wave & 1, wc = wave >> 1;  // rows 64*wr.., column tiles kWct*wc..
  const int64_t row0 = (int64_t)blockIdx.x * kApRows;
  const int nsteps = d_model / kApK;
  const int st0 = blockIdx.y * steps_per_split;
  const int st1 = min(st0 + steps_per_split, nsteps);

  // Pair p = tid + j*kApThreads covers tile p >> 6, lane p & 63: slots
  // ((p >> 6) * 2 + ks) * 64 + (p & 63) for ks = 0, 1.  Element offsets at K
  // step 0; a pair of a row past M reads row M-1 instead: that row's products
  // only reach output rows that are never stored, and the loads stay
  // unconditional.
  int64_t aoff[kPerA];
  int64_t boff[kPerB];
#pragma unroll
  for (int j = 0; j < kPerA; ++j) {
    const int p = tid + j * kApThreads;
    const int64_t row = min(row0 + (p >> 6) * 16 + (p & 15), (int64_t)M - 1);
    aoff[j] = row * d_model + 16 * ((p >> 4) & 3);
  }
#pragma unroll
  for (int j = 0; j < kPerB; ++j) {
    // pairs past kPairsB (Dc = 192) load the last pair again and store nothing
    const int p = min(tid + j * kApThreads, kPairsB - 1);
    const int col = (p >> 6) * 16 + (p & 15);
    boff[j] = (int64_t)col * d_model + 16 * ((p >> 4) & 3);
  }
  auto slot = [&](int j, int ks) { return (((tid + j * kApThreads) >> 6) * 2 + ks) * 64 + (tid & 63); };

  // D register stages: stage u holds the step st0 + u (mod D) loaded D steps
  // ahead of its use, so D steps of MFMA work cover each load's latency.
  i32x4 ra[D][kPerA][2], rb[D][kPerB][2];
  auto gload = [&](int u, int st) {
    const int64_t k0 = (int64_t)st * kApK;
#pragma unroll
    for (int j = 0; j < kPerA; ++j) {
      ra[u][j][0] = ld16(h + aoff[j] + k0);
      ra[u][j][1] = ld16(h + aoff[j] + k0 + 8);
    }
#pragma unroll
    for (int j = 0; j < kPerB; ++j) {
      rb[u][j][0] = ld16(w_enc + boff[j] + k0);
      rb[u][j][1] = ld16(w_enc + boff[j] + k0 + 8);
    }
  };
  auto lstore = [&](int buf, int u) {
#pragma unroll
    for (int j = 0; j < kPerA; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) tile[buf][slot(j, ks)] = ra[u][j][ks];
#pragma unroll
    for (int j = 0; j < kPerB; ++j) {
      if (kPerB * kApThreads != kPairsB && tid + j * kApThreads >= kPairsB) continue;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) tile[buf][kApSlotsA + slot(j, ks)] = rb[u][j][ks];
    }
  };

  f32x4 acc[4][kWct];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWct; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[4], b[kWct];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = __builtin_bit_cast(bf16x8, tile[buf][((4 * wr + i) * 2 + ks) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < kWct; ++j)
        b[j] = __builtin_bit_cast(bf16x8, tile[buf][kApSlotsA + ((kWct * wc + j) * 2 + ks) * 64 + lane]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kWct; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Loads and LDS stores are unconditional, so the compiler's wait counts
  // track exactly the D steps in flight: a load past the split's last step
  // re-reads that step (in bounds), and the last step's store fills the buffer
  // no wave reads again.
#pragma unroll
  for (int u = 0; u < D; ++u) gload(u, min(st0 + u, st1 - 1));
  lstore(0, 0);
  __syncthreads();
  auto step = [&](int u, int st) {
    const int buf = (st - st0) & 1;
    // stage u's step is in LDS already (stored before the last barrier)
    gload(u, min(st + D, st1 - 1));
    // keep the loads first: the scheduler would otherwise sink them below the
    // step's MFMAs, shortening the distance they run ahead by a step
    __builtin_amdgcn_sched_barrier(0);
    compute(buf);
    // The other buffer was last read in the previous step, which every wave
    // finished before the barrier that ended it.
    lstore(buf ^ 1, (u + 1) % D);
    __syncthreads();
  };
  // Whole groups of D steps in the loop, the rest after it: no path through
  // the loop skips a store, so no wait drains the loads in flight.
  int base = st0;
  for (; base + D <= st1; base += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(u, base + u);
  }
#pragma unroll
  for (int u = 0; u + 1 < D; ++u)
    if (base + u < st1) step(u, base + u);

  // acc[i][j][e]: row 64*wr + 16*i + 4*(lane >> 4) + e, column 16*(kWct*wc + j) + (lane & 15).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = row0 + 64 * wr + 16 * i + 4 * (lane >> 4) + e;
      if (row >= M) continue;
      if (part) {
        float* out = part + ((int64_t)blockIdx.y * M + row) * DC + (lane & 15);
#pragma unroll
        for (int j = 0; j < kWct; ++j) out[16 * (kWct * wc + j)] = acc[i][j][e];
      } else {
        uint16_t* out = latent + dst[row] * DC + (lane & 15);
#pragma unroll
        for (int j = 0; j < kWct; ++j) out[16 * (kWct * wc + j)] = bf16_rne(acc[i][j][e]);
      }
    }
  }
}

// Sum of the S partial tiles, rounded to bf16 and stored at dst_row.  A
// workgroup covers R rows; thread (r, g, quad) adds splits g, g + G, g + 2G,
// ... in increasing order for four consecutive columns of its row, and thread
// (r, 0, quad) then adds the G group sums in order g = 0 .. G-1.  The order
// depends only on S and G, never on scheduling.
// F8: the row is stored as E4M3 codes with one fp32 scale per 128 values
// counted from the row's start (the last block shorter when Dc is not a
// multiple of 128; the block's largest magnitude / 448, or 1 for an all-zero
// block); a block is up to 32 quads held by 32 consecutive lanes.  A row's
// quads sit on QP lanes, the next power of two of Dc / 4 (Dc = 192: 48 quads
// on 64 lanes, the last 16 idle), so each block starts on a 32-lane boundary.
template <int DC, bool F8>
__global__ __launch_bounds__(1024) void append_reduce_kernel(const float* __restrict__ part, int32_t S, int32_t G,
                                                             int32_t M, const int64_t* __restrict__ dst,
                                                             uint16_t* __restrict__ latent, float* __restrict__ c_scale) {
  constexpr int QD = DC / 4;
  constexpr int QP = append_row_lanes(DC);
  __shared__ f32x4 red[1024];
  const int tid = threadIdx.x;
  const int qp = tid % QP, g = (tid / QP) % G;
  const int q = qp < QD ? qp : QD - 1;  // idle lanes read the last quad and store nothing
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / (QP * G)) + tid / (QP * G);
  const bool live = row < M;
  const int64_t plane = (int64_t)M * DC;
  const float* p = part + (live ? row : 0) * DC + 4 * q;
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = g;
  if (live) {
    for (; s + 7 * G < S; s += 8 * G) {  // eight independent loads in flight
      f32x4 u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = *reinterpret_cast<const f32x4*>(p + (s + j * G) * plane);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += u[j][e];
    }
    for (; s < S; s += G) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(p + s * plane);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += u[e];
    }
  }
  if (G > 1) {
    red[tid] = v;
    __syncthreads();
    if (g != 0) return;
    for (int j = 1; j < G; ++j) {
      const f32x4 u = red[tid + j * QP];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += u[e];
    }
  }
  if (!live) return;  // uniform over each row's lanes
  const bool own = qp < QD;
  if constexpr (F8) {
    float am = own ? fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))) : 0.f;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (!own) return;
    const float sc = am > 0.f ? am / 448.f : 1.f;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= e4m3_rne(v[e] / sc) << (8 * e);
    const int64_t r = dst[row];
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(latent) + r * DC + 4 * q) = word;
    if ((q & 31) == 0) c_scale[r * ((DC + 127) / 128) + q / 32] = sc;
  } else {
    if (!own) return;
    const uint32_t lo = (uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16);
    const uint32_t hi = (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16);
    *reinterpret_cast<i32x2*>(latent + dst[row] * DC + 4 * q) = i32x2{(int)lo, (int)hi};
  }
}

}  // namespace

int32_t append_splits(int32_t M, int32_t d_model) {
  const int32_t nsteps = d_model / kApK;
  const int32_t row_blocks = (M + kApRows - 1) / kApRows;
  // Enough workgroups to cover the 256 compute units (one K step per split at
  // the least); one split writes the cache directly.
  int32_t s = (256 + row_blocks - 1) / row_blocks;
  if (s > nsteps) s = nsteps;
  const int32_t per = (nsteps + s - 1) / s;
  return (nsteps + per - 1) / per;  // no empty split
}

hipError_t launch_latent_append(const uint16_t* h, const uint16_t* w_enc, const int64_t* dst, int32_t M,
                                int32_t d_model, int32_t Dc, float* part, uint16_t* latent, bool fp8, float* c_scale,
                                hipStream_t stream) {
  constexpr int D = kApDepth;
  const int32_t S = append_splits(M, d_model);
  const int32_t nsteps = d_model / kApK;
  const int32_t per = (nsteps + S - 1) / S;
  const dim3 grid((unsigned)((M + kApRows - 1) / kApRows), (unsigned)S);
  float* p = S > 1 || fp8 ? part : nullptr;  // fp8 output always goes through the split sum
  hipError_t e;
  if (Dc == 256)
    e = launch_kernel(append_gemm_kernel<256, D>, grid, dim3(kApThreads), 0, stream, h, w_enc, dst, M, d_model, per,
                      p, latent);
  else if (Dc == 192)
    e = launch_kernel(append_gemm_kernel<192, D>, grid, dim3(kApThreads), 0, stream, h, w_enc, dst, M, d_model, per,
                      p, latent);
  else
    e = launch_kernel(append_gemm_kernel<128, D>, grid, dim3(kApThreads), 0, stream, h, w_enc, dst, M, d_model, per,
                      p, latent);
  if (e != hipSuccess || !p) return e;
  // G split groups per row, each summing at most eight splits (G <= 16); a
  // workgroup holds 256 threads or one row's Dc/4 * G, whichever is larger.
  int32_t G = 1;
  while (G < 16 && G * 8 < S) G *= 2;
  const int32_t per_row = append_row_lanes(Dc) * G;
  const int32_t rows = per_row >= 256 ? 1 : 256 / per_row;
  const dim3 grid_r((unsigned)((M + rows - 1) / rows)), block_r((unsigned)(rows * per_row));
  const float* cp = part;
  if (fp8) {
    if (Dc == 256)
      return launch_kernel(append_reduce_kernel<256, true>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent,
                           c_scale);
    if (Dc == 192)
      return launch_kernel(append_reduce_kernel<192, true>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent,
                           c_scale);
    return launch_kernel(append_reduce_kernel<128, true>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent, c_scale);
  }
  if (Dc == 256)
    return launch_kernel(append_reduce_kernel<256, false>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent,
                         c_scale);
  if (Dc == 192)
    return launch_kernel(append_reduce_kernel<192, false>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent,
                         c_scale);
  return launch_kernel(append_reduce_kernel<128, false>, grid_r, block_r, 0, stream, cp, S, G, M, dst, latent, c_scale);
}

}  // namespace li
