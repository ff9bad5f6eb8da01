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
// small Dc (128 or 256) and a long K, so it runs on bf16 MFMA
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

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// LDS holds each K step's tiles in MFMA fragment order: slot
// ((t * 2 + ks) * 64 + lane) is the 16 bytes that `lane` feeds to the MFMA of
// 16-row tile t and 32-wide K block ks (row t*16 + (lane & 15), K elements
// ks*32 + 8*(lane >> 4) .. +7), so fragment reads are consecutive per wave.
// The producer of a slot is the thread with that slot's index, so the LDS
// writes are consecutive too; its global read covers 64 contiguous bytes of a
// row per four lanes.
template <int DC>
__global__ __launch_bounds__(kApThreads, 1) void append_gemm_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_enc, const int64_t* __restrict__ dst,
    int32_t M, int32_t d_model, int32_t steps_per_split, float* __restrict__ part,
    uint16_t* __restrict__ latent) {
  constexpr int kSlotsB = DC / 16 * 2 * 64;
  constexpr int kPerA = kApSlotsA / kApThreads;
  constexpr int kPerB = kSlotsB / kApThreads;
  constexpr int kWct = DC / 16 / 4;  // 16-column tiles per wave
  static_assert(kPerA * kApThreads == kApSlotsA && kPerB * kApThreads == kSlotsB, "tile split");
  __shared__ i32x4 tile[2][kApSlotsA + kSlotsB];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wr = wave & 1, wc = wave >> 1;  // rows 64*wr.., column tiles kWct*wc..
  const int64_t row0 = (int64_t)blockIdx.x * kApRows;
  const int nsteps = d_model / kApK;
  const int st0 = blockIdx.y * steps_per_split;
  const int st1 = min(st0 + steps_per_split, nsteps);

  // Element offsets of this thread's slots (at K step 0).
  int64_t aoff[kPerA];
  bool aok[kPerA];
  int64_t boff[kPerB];
#pragma unroll
  for (int j = 0; j < kPerA; ++j) {
    const int q = tid + j * kApThreads;
    const int64_t row = row0 + (q >> 7) * 16 + (q & 15);
    const int c = ((q >> 6) & 1) * 4 + ((q >> 4) & 3);
    aok[j] = row < M;
    aoff[j] = (aok[j] ? row : 0) * d_model + c * 8;
  }
#pragma unroll
  for (int j = 0; j < kPerB; ++j) {
    const int q = tid + j * kApThreads;
    const int col = (q >> 7) * 16 + (q & 15);
    const int c = ((q >> 6) & 1) * 4 + ((q >> 4) & 3);
    boff[j] = (int64_t)col * d_model + c * 8;
  }

  i32x4 ra[kPerA], rb[kPerB];
  auto gload = [&](int st) {
    const int64_t k0 = (int64_t)st * kApK;
#pragma unroll
    for (int j = 0; j < kPerA; ++j) ra[j] = aok[j] ? ld16(h + aoff[j] + k0) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kPerB; ++j) rb[j] = ld16(w_enc + boff[j] + k0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kPerA; ++j) tile[buf][tid + j * kApThreads] = ra[j];
#pragma unroll
    for (int j = 0; j < kPerB; ++j) tile[buf][kApSlotsA + tid + j * kApThreads] = rb[j];
  };

  f32x4 acc[4][kWct];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWct; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(st0);
  lstore(0);
  __syncthreads();
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    const bool more = st + 1 < st1;
    if (more) gload(st + 1);
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
        for (int j = 0; j < kWct; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // The other buffer was last read in the previous step, which every wave
    // finished before the barrier that ended it.
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

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

// Sum of the S partial tiles in split order, rounded to bf16, at dst_row.
// One thread per four consecutive columns of a row.
template <int DC>
__global__ __launch_bounds__(256) void append_reduce_kernel(const float* __restrict__ part, int32_t S, int32_t M,
                                                            const int64_t* __restrict__ dst,
                                                            uint16_t* __restrict__ latent) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / (DC / 4);
  const int c = (int)(t % (DC / 4)) * 4;
  if (row >= M) return;
  const int64_t plane = (int64_t)M * DC;
  const float* p = part + row * DC + c;
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  for (int s = 1; s < S; ++s) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p + s * plane);
    v[0] += u[0];
    v[1] += u[1];
    v[2] += u[2];
    v[3] += u[3];
  }
  const uint32_t lo = (uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16);
  const uint32_t hi = (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16);
  *reinterpret_cast<i32x2*>(latent + dst[row] * DC + c) = i32x2{(int)lo, (int)hi};
}

}  // namespace

int32_t append_splits(int32_t M, int32_t d_model) {
  const int32_t nsteps = d_model / kApK;
  const int32_t row_blocks = (M + kApRows - 1) / kApRows;
  // Enough workgroups to cover the 256 compute units, each split keeping at
  // least two K steps; one split writes the cache directly.
  int32_t s = (256 + row_blocks - 1) / row_blocks;
  const int32_t cap = nsteps / 2 > 1 ? nsteps / 2 : 1;
  if (s > cap) s = cap;
  const int32_t per = (nsteps + s - 1) / s;
  return (nsteps + per - 1) / per;  // no empty split
}

hipError_t launch_latent_append(const uint16_t* h, const uint16_t* w_enc, const int64_t* dst, int32_t M,
                                int32_t d_model, int32_t Dc, float* part, uint16_t* latent, hipStream_t stream) {
  const int32_t S = append_splits(M, d_model);
  const int32_t nsteps = d_model / kApK;
  const int32_t per = (nsteps + S - 1) / S;
  const dim3 grid((unsigned)((M + kApRows - 1) / kApRows), (unsigned)S);
  float* p = S > 1 ? part : nullptr;
  hipError_t e;
  if (Dc == 256)
    e = launch_kernel(append_gemm_kernel<256>, grid, dim3(kApThreads), 0, stream, h, w_enc, dst, M, d_model, per, p,
                      latent);
  else
    e = launch_kernel(append_gemm_kernel<128>, grid, dim3(kApThreads), 0, stream, h, w_enc, dst, M, d_model, per, p,
                      latent);
  if (e != hipSuccess || S == 1) return e;
  const unsigned blocks = (unsigned)(((int64_t)M * (Dc / 4) + 255) / 256);
  if (Dc == 256)
    return launch_kernel(append_reduce_kernel<256>, dim3(blocks), dim3(256), 0, stream, (const float*)part, S, M, dst,
                         latent);
  return launch_kernel(append_reduce_kernel<128>, dim3(blocks), dim3(256), 0, stream, (const float*)part, S, M, dst,
                       latent);
}

}  // namespace li
