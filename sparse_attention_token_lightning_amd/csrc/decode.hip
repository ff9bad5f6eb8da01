// Decode scan of the lightning indexer on gfx950.
//
// For each request b (one query token) and each cached position s < L_b:
//   S[s] = k_scale[s] * sum_h w[b][h] * ReLU(q[b][h] . k_hat[s])
// (one score per visible position, "IndexCache: Cross-Layer Index Reuse for
// Sparse Attention", Symbol Map; positive per-token scales commute with ReLU).
//
// Work per key is 64 heads x 128 dims = 16 KFLOP against 132 bytes (fp8 + its
// fp32 scale), i.e. ~124 FLOP/B: above what the VALU can feed at HBM speed, so
// the per-head contraction runs on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16) and the kernel stays HBM-bound.
//
// Mapping: the 64 query heads are the MFMA's M (two 32-row blocks held in
// registers for the whole kernel), 32 consecutive keys are its N, and the 128
// dims are its K.  Lane l works on key (l & 31) and dims 64*(l >> 5) .. +63 of
// it, so each lane streams one contiguous 64-byte (fp8) or 128-byte (bf16)
// half row with 16-byte loads and converts fp8 -> bf16 exactly in registers.
// The contraction index is summed, so A and B use the same dims-to-lane
// assignment and any such assignment is valid.  The MFMA result leaves each
// lane 16 heads of its key per block: ReLU, the head weight and the sum over
// the lane's 32 heads happen in registers, and one cross-half shuffle finishes
// the 64-head sum.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kDecWaves = 4;       // waves per workgroup
constexpr int kTile = 32;          // keys per MFMA tile

template <bool FP8>
__global__ __launch_bounds__(256) void decode_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kc,
    const float* __restrict__ k_scale, const int64_t* __restrict__ kv_off, int H,
    int tiles_per_wave, float* __restrict__ scores) {
  constexpr int NV = FP8 ? 4 : 8;              // 16-byte vectors per lane per tile
  constexpr int kRowBytes = FP8 ? 128 : 256;   // one key row
  const int b = blockIdx.y;
  const int64_t off = kv_off[b];
  const int64_t L = kv_off[b + 1] - off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int64_t chunk = (int64_t)kDecWaves * tiles_per_wave * kTile;
  int64_t t0 = (int64_t)blockIdx.x * chunk + (int64_t)wave * kTile;
  if (t0 >= L) return;

  // Query heads as MFMA A operand: row = head (hb*32 + col), dims 64g + 8j .. +7.
  bf16x8 qa[2][8];
  float wl[2][16];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int row = hb * 32 + col;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      i32x4 v = {0, 0, 0, 0};
      if (row < H) v = ld16(q + ((int64_t)b * H + row) * 128 + 64 * g + 8 * j);
      qa[hb][j] = __builtin_bit_cast(bf16x8, v);
    }
    // The heads whose results this lane holds: rows 8*(r/4) + 4*g + r%4 of the block.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      wl[hb][r] = head < H ? w[(int64_t)b * H + head] : 0.0f;
    }
  }

  const uint8_t* kbase = kc + (off * kRowBytes) + (FP8 ? 64 : 128) * g;
  auto load_tile = [&](i32x4 (&raw)[NV], int64_t tt0) {
    int64_t s = tt0 + col;
    s = s < L ? s : L - 1;
    const uint8_t* p = kbase + s * kRowBytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = ld16(p + 16 * v);
  };

  i32x4 cur[NV], nxt[NV];
  load_tile(cur, t0);
  for (int it = 0;;) {
    const int64_t t1 = t0 + (int64_t)kDecWaves * kTile;
    const bool has_next = (++it < tiles_per_wave) && (t1 < L);
    if (has_next) load_tile(nxt, t1);

    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 kb;
      if constexpr (FP8) {
        const i32x4 v = cur[j >> 1];
        kb = (j & 1) ? fp8x8_to_bf16x8(v.z, v.w) : fp8x8_to_bf16x8(v.x, v.y);
      } else {
        kb = __builtin_bit_cast(bf16x8, cur[j]);
      }
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][j], kb, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][j], kb, a1, 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(wl[0][r], fmaxf(a0[r], 0.0f), part);
      part = fmaf(wl[1][r], fmaxf(a1[r], 0.0f), part);
    }
    part += __shfl_xor(part, 32, 64);
    const int64_t s = t0 + col;
    if (g == 0 && s < L) {
      const float sc = k_scale ? k_scale[off + s] : 1.0f;
      scores[off + s] = part * sc;
    }
    if (!has_next) break;
#pragma unroll
    for (int v = 0; v < NV; ++v) cur[v] = nxt[v];
    t0 = t1;
  }
}

}  // namespace

hipError_t launch_decode_score(const uint16_t* q, const float* w, const void* kc, bool kc_fp8,
                               const float* k_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t H, float* scores,
                               hipStream_t stream) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  // Tiles per wave: enough workgroups to fill 256 CUs several times over, but
  // long enough runs that each workgroup's one-off query load is amortised.
  int64_t tpw = n_tok / ((int64_t)2048 * kDecWaves * kTile);
  tpw = tpw < 1 ? 1 : (tpw > 16 ? 16 : tpw);
  const int64_t chunk = (int64_t)kDecWaves * tpw * kTile;
  dim3 grid((unsigned)((max_len + chunk - 1) / chunk), (unsigned)B);
  dim3 block(64 * kDecWaves);
  if (kc_fp8)
    decode_score_kernel<true><<<grid, block, 0, stream>>>(
        q, w, (const uint8_t*)kc, k_scale, kv_off, H, (int)tpw, scores);
  else
    decode_score_kernel<false><<<grid, block, 0, stream>>>(
        q, w, (const uint8_t*)kc, k_scale, kv_off, H, (int)tpw, scores);
  return hipGetLastError();
}

}  // namespace li
