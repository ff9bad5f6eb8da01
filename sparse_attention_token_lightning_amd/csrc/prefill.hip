// Prefill scan of the lightning indexer on gfx950: T new query tokens of one
// sequence against its L-token key cache, causal.
//
//   S[t][s] = q_scale[t] * k_scale[s] * sum_h w[t][h] * ReLU(q_hat[t][h] . k_hat[s]),
//   visible iff s <= qpos0 + t
//
// This is a real dense contraction (M = T*64 query-head rows, N = L keys,
// K = 128) with fp8 operands, so it runs on the fp8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, OCP E4M3 for both operands), with the
// ReLU-weighted head reduction, the two scales and the causal mask fused into
// the epilogue; fully masked key tiles are never computed.
//
// Mapping: a wave owns two query tokens (2 x 64 heads = four 32-row M blocks,
// held in registers) and walks the visible keys 32 at a time.  Lane l works on
// key (l & 31) and dims 64*(l >> 5) .. +63 of it; the head sum is finished in
// registers plus one cross-half shuffle, as in the decode scan.
//
// A wave owns whole rows, so it also builds each row's level-0 selection
// histogram in LDS and finds the row's threshold bin for the top-k itself.
#include "li_device.h"
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTokPerWave = 2;
constexpr int kPfTokPerBlock = kPfWaves * kPfTokPerWave;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 ld32(const uint8_t* p) {
  const i32x4 x = ld16(p), y = ld16(p + 16);
  i32x8 r = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
  return r;
}

// The wave's lanes each own 32 consecutive bins of a row's histogram (from the
// top); the lane whose bins cross the kk-th largest key writes the threshold.
__device__ void wave_find_bin(const uint32_t* hist, uint32_t kk, uint32_t* thr) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kSelBins / 64;
  uint32_t sum = 0;
  for (int i = 0; i < PER; ++i) sum += hist[kSelBins - 1 - (lane * PER + i)];
  uint32_t run = wave_incl_scan(sum) - sum;
  for (int i = 0; i < PER; ++i) {
    const uint32_t h = hist[kSelBins - 1 - (lane * PER + i)];
    if (run < kk && run + h >= kk) {
      thr[0] = (uint32_t)(kSelBins - 1 - (lane * PER + i));
      thr[1] = run;
      thr[2] = h;
      thr[3] = 1u;
    }
    run += h;
  }
}

__global__ __launch_bounds__(256) void prefill_score_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kc, const float* __restrict__ k_scale, int T, int L, int qpos0,
    int H, int k, int fill_masked, float* __restrict__ scores, uint32_t* __restrict__ thr) {
  __shared__ uint32_t phist[kPfWaves][kPfTokPerWave][kSelBins];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int t_base = (blockIdx.x * kPfWaves + wave) * kPfTokPerWave;
  for (int i = lane; i < kPfTokPerWave * kSelBins; i += 64) (&phist[wave][0][0])[i] = 0;
  __syncthreads();
  const int nt = t_base >= T ? 0 : ((T - t_base) < kPfTokPerWave ? (T - t_base) : kPfTokPerWave);

  i32x8 qa[kPfTokPerWave][2][2];
  float wl[kPfTokPerWave][2][16];
  float sq[kPfTokPerWave];
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk) {
    const int t = nt > 0 ? t_base + (tk < nt ? tk : 0) : 0;  // always a valid row
    sq[tk] = q_scale ? q_scale[t] : 1.0f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int row = hb * 32 + col;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        i32x8 v = {};
        if (row < H) v = ld32(q + ((int64_t)t * H + row) * 128 + 64 * g + 32 * j);
        qa[tk][hb][j] = v;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int head = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        wl[tk][hb][r] = head < H ? w[(int64_t)t * H + head] : 0.0f;
      }
    }
  }

  const int vis_end = qpos0 + t_base + nt;  // exclusive end of the last token's visible range
  const int n_tiles = nt > 0 ? (vis_end + 31) / 32 : 0;
  const uint8_t* kbase = kc + 64 * g;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int s = kt * 32 + col;
    const int srow = s < L ? s : L - 1;
    const i32x8 kb0 = ld32(kbase + (int64_t)srow * 128);
    const i32x8 kb1 = ld32(kbase + (int64_t)srow * 128 + 32);
    const float sk = k_scale ? k_scale[srow] : 1.0f;
#pragma unroll
    for (int tk = 0; tk < kPfTokPerWave; ++tk) {
      if (tk < nt) {
        f32x16 a0 = {}, a1 = {};
        a0 = mfma_fp8(qa[tk][0][0], kb0, a0);
        a1 = mfma_fp8(qa[tk][1][0], kb0, a1);
        a0 = mfma_fp8(qa[tk][0][1], kb1, a0);
        a1 = mfma_fp8(qa[tk][1][1], kb1, a1);
        float part = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          part = fmaf(wl[tk][0][r], relu(a0[r]), part);
          part = fmaf(wl[tk][1][r], relu(a1[r]), part);
        }
        part = sum_halves(part);
        const int t = t_base + tk;
        if (g == 0 && s < L) {
          if (s <= qpos0 + t) {
            const float val = part * sq[tk] * sk;
            scores[(int64_t)t * L + s] = val;
            atomicAdd(&phist[wave][tk][score_key(val) >> kSelShift], 1u);
          } else {
            scores[(int64_t)t * L + s] = -INFINITY;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int tk = 0; tk < nt; ++tk) {
    const int t = t_base + tk;
    if (qpos0 + t + 1 > k) wave_find_bin(phist[wave][tk], (uint32_t)k, thr + (int64_t)t * 4);
  }
  if (fill_masked) {
    for (int tk = 0; tk < nt; ++tk) {
      const int t = t_base + tk;
      for (int s = n_tiles * 32 + lane; s < L; s += 64) scores[(int64_t)t * L + s] = -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_prefill_score(const uint8_t* q, const float* q_scale, const float* w,
                                const uint8_t* kc, const float* k_scale, int32_t T, int32_t L,
                                int32_t qpos0, int32_t H, int32_t k, bool fill_masked,
                                float* scores, const SelWs& sel, hipStream_t stream) {
  if (T <= 0 || L <= 0) return hipSuccess;
  dim3 grid((unsigned)((T + kPfTokPerBlock - 1) / kPfTokPerBlock));
  prefill_score_kernel<<<grid, dim3(64 * kPfWaves), 0, stream>>>(
      q, q_scale, w, kc, k_scale, T, L, qpos0, H, k, fill_masked ? 1 : 0, scores, sel.thr);
  return hipGetLastError();
}

}  // namespace li
