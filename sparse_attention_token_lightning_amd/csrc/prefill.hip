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

constexpr int kPfStages = 3;  // key tiles per wave in the register ring

__global__ __launch_bounds__(256) void prefill_score_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kc, const float* __restrict__ k_scale, int T, int L, int qpos0,
    int H, int k, int fill_masked, float* __restrict__ scores, uint32_t* __restrict__ thr) {
  __shared__ uint32_t phist[kPfWaves][kPfTokPerWave][kSelBins];
  // Head weights of the block's tokens.  In the MFMA result a lane holds heads
  // 8*(r/4) + 4*g + r%4 (+32 per row block): every lane of a half reads the
  // same four consecutive weights, so these reads are LDS broadcasts.
  __shared__ float wsh[kPfTokPerBlock][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int t_base = (blockIdx.x * kPfWaves + wave) * kPfTokPerWave;
  const int nt = t_base >= T ? 0 : ((T - t_base) < kPfTokPerWave ? (T - t_base) : kPfTokPerWave);
  // Token slot tk computes row trow[tk]; slots past the end of the chunk
  // repeat the wave's first token (so their stores rewrite identical values)
  // and are never counted in a histogram.
  int trow[kPfTokPerWave];
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk) trow[tk] = nt > 0 ? t_base + (tk < nt ? tk : 0) : 0;

  for (int i = lane; i < kPfTokPerWave * kSelBins; i += 64) (&phist[wave][0][0])[i] = 0;
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk)
    wsh[wave * kPfTokPerWave + tk][lane] = lane < H ? w[(int64_t)trow[tk] * H + lane] : 0.0f;

  i32x8 qa[kPfTokPerWave][2][2];
  float sq[kPfTokPerWave];
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk) {
    sq[tk] = q_scale ? q_scale[trow[tk]] : 1.0f;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int row = hb * 32 + col;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        i32x8 v = {};
        if (row < H) v = ld32(q + ((int64_t)trow[tk] * H + row) * 128 + 64 * g + 32 * j);
        qa[tk][hb][j] = v;
      }
    }
  }
  __syncthreads();

  const int vis_end = qpos0 + t_base + nt;  // exclusive end of the last token's visible range
  const int n_tiles = nt > 0 ? (vis_end + 31) / 32 : 0;
  const uint8_t* kbase = kc + 64 * g;
  // Key row of tile `it` for this lane, clamped into the cache: a lane past
  // the end recomputes row L-1 and rewrites that row's own score.
  auto key_row = [&](int it) {
    const int s = it * 32 + col;
    return s < L ? s : L - 1;
  };
  auto load_tile = [&](i32x8 (&kb)[2], float& sk, int it) {
    const int srow = key_row(it);
    const uint8_t* p = kbase + (int64_t)srow * 128;
    kb[0] = ld32(p);
    kb[1] = ld32(p + 32);
    sk = k_scale ? k_scale[srow] : 1.0f;
  };
  auto compute = [&](const i32x8 (&kb)[2], float sk, int it, bool live) {
    const int s = it * 32 + col;
    const int srow = key_row(it);
    f32x16 acc[kPfTokPerWave][2];
#pragma unroll
    for (int tk = 0; tk < kPfTokPerWave; ++tk) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x16 a = {};
        a = mfma_fp8(qa[tk][hb][0], kb[0], a);
        acc[tk][hb] = mfma_fp8(qa[tk][hb][1], kb[1], a);
      }
    }
#pragma unroll
    for (int tk = 0; tk < kPfTokPerWave; ++tk) {
      const float* wt = &wsh[wave * kPfTokPerWave + tk][4 * g];
      float part = 0.0f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(wt + hb * 32 + 8 * r4);
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wv[i], relu(acc[tk][hb][4 * r4 + i]), part);
        }
      }
      part = sum_halves(part);
      const int t = trow[tk];
      const bool vis = srow <= qpos0 + t;
      const float val = vis ? part * sq[tk] * sk : -INFINITY;
      // Straight-line store (both halves write the same value) so the loads
      // of the next tiles stay in flight.
      scores[(int64_t)t * L + srow] = val;
      // (an LDS-only branch)
      if (live && tk < nt && g == 0 && s < L && vis)
        atomicAdd(&phist[wave][tk][score_key(val) >> kSelShift], 1u);
    }
  };

  if (n_tiles > 0) {
    i32x8 buf[kPfStages][2];
    float skb[kPfStages];
#pragma unroll
    for (int st = 0; st < kPfStages - 1; ++st) load_tile(buf[st], skb[st], st < n_tiles ? st : n_tiles - 1);
    const int nit = (n_tiles + kPfStages - 1) / kPfStages * kPfStages;
    for (int base = 0; base < nit; base += kPfStages) {
#pragma unroll
      for (int st = 0; st < kPfStages; ++st) {
        const int it = base + st;
        const int nx = it + kPfStages - 1;
        load_tile(buf[(st + kPfStages - 1) % kPfStages], skb[(st + kPfStages - 1) % kPfStages],
                  nx < n_tiles ? nx : n_tiles - 1);
        compute(buf[st], skb[st], it < n_tiles ? it : n_tiles - 1, it < n_tiles);
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
