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
// it and converts fp8 -> bf16 exactly in registers.  bf16 keys: each lane
// streams its 128-byte half row with 16-byte loads.  fp8 keys: every 16-byte
// load instruction of a wave covers 8 whole key rows (1 KB contiguous), read
// with the non-temporal hint (a stream of whole lines runs about 14% faster
// with it; a line split over several instructions runs far slower), and the
// wave turns the 4 KB tile into the per-key layout through its own LDS slice.
// The contraction index is summed, so A and B use the same dims-to-lane
// assignment and any such assignment is valid.  The MFMA result leaves each
// lane 16 heads of its key per block: ReLU, the head weight and the sum over
// the lane's 32 heads happen in registers, and one cross-half shuffle finishes
// the 64-head sum.
//
// Latency hiding: each wave keeps 3 (fp8) or 2 (bf16) key tiles in flight in
// registers while it computes a fourth (a ring indexed at compile time, so no
// register copies force early waits), together with their per-token scales.
//
// Scores collect in LDS and leave in one coalesced burst per workgroup: a
// 4-byte store per key interleaved with the key stream costs several times its
// own share of HBM time.
//
// The selection's first radix level is fused in: every score also lands in a
// per-workgroup LDS histogram of its top 11 key bits, stored as that
// workgroup's partial of the request's histogram (plain stores: dozens of
// workgroups adding into the same hot bins with atomics serialise badly).
#include "li_device.h"
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kDecWaves = 4;  // waves per workgroup
constexpr int kTile = 32;     // keys per MFMA tile
constexpr int kStagesFp8 = 4;   // key-tile buffers per wave (fp8 keys)
constexpr int kStagesBf16 = 3;  // (bf16 keys: twice the registers per tile)
constexpr int kDecMaxTpw = 64;  // tiles per wave at most
constexpr int kDecMaxChunk = kDecWaves * kDecMaxTpw * kTile;  // positions per workgroup at most

template <bool FP8>
__global__ __launch_bounds__(256) void decode_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kc,
    const float* __restrict__ k_scale, const int64_t* __restrict__ kv_off, int H,
    int tiles_per_wave, int k, float* __restrict__ scores, SelWs sel) {
  constexpr int NV = FP8 ? 4 : 8;             // 16-byte vectors per lane per tile
  constexpr int kRowBytes = FP8 ? 128 : 256;  // one key row
  constexpr int kStages = FP8 ? kStagesFp8 : kStagesBf16;
  __shared__ __attribute__((aligned(16))) uint32_t lhist[kSelBins + 128];  // + spare words for the bucket epilogue
  // The workgroup's scores as order-preserving keys (score_key), written to
  // HBM in one burst at the end: small writes interleaved with the key stream
  // cost far more read bandwidth than their own size.
  __shared__ __attribute__((aligned(16))) uint32_t ssc[kDecMaxChunk];
  __shared__ uint32_t wsum[kDecWaves];
  __shared__ uint32_t sh_floor[2];
  // fp8: each wave's key tile (32 rows x 128 B) on its way from the
  // row-contiguous load layout to the MFMA operand layout.
  __shared__ __attribute__((aligned(16))) uint8_t ktl[FP8 ? kDecWaves : 1][FP8 ? kTile * 128 : 16];

  const int b = blockIdx.y;
  const int64_t off = kv_off[b];
  const int64_t L = kv_off[b + 1] - off;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int col = lane & 31, g = lane >> 5;
  const int64_t chunk = (int64_t)kDecWaves * tiles_per_wave * kTile;
  const int64_t wg0 = (int64_t)blockIdx.x * chunk;
  if (wg0 >= L) return;  // whole workgroup: no key of this request here
  const bool select = L > k;
  for (int i = tid; i < kSelBins; i += 256) lhist[i] = 0;
  // The segmented top-k kernel that follows counts finished segments per request.
  if (select && !sel.bucket && blockIdx.x == 0 && tid == 0) sel.done[b] = 0u;

  // Query heads as MFMA A operand: row = head (hb*32 + col), dims 64g + 8j .. +7.
  bf16x8 qa[2][8];
  float wl[2][16];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int row = hb * 32 + col;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // Clamped, unconditional load (rows past H are zeroed afterwards): a
      // load under a branch would be waited for before the next one issues.
      i32x4 v = ld16(q + ((int64_t)b * H + (row < H ? row : H - 1)) * 128 + 64 * g + 8 * j);
      if (row >= H) v = i32x4{0, 0, 0, 0};
      qa[hb][j] = __builtin_bit_cast(bf16x8, v);
    }
    // The heads whose results this lane holds: rows 8*(r/4) + 4*g + r%4 of the block.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      const float wv = w[(int64_t)b * H + (head < H ? head : H - 1)];
      wl[hb][r] = head < H ? wv : 0.0f;
    }
  }
  __syncthreads();

  // This wave's tiles: it = 0 .. nt-1 at tokens wg0 + 32*(wave + 4*it).
  const int64_t w0 = wg0 + (int64_t)wave * kTile;
  int nt = 0;
  if (w0 < L) {
    const int64_t t = (L - w0 + (int64_t)kDecWaves * kTile - 1) / ((int64_t)kDecWaves * kTile);
    nt = (int)(t < tiles_per_wave ? t : tiles_per_wave);
  }
  const uint8_t* kbase = kc + off * kRowBytes + (FP8 ? 0 : 128 * g);
  // Positions relative to the request fit in 32 bits (max_len is an int32).
  const int w0i = (int)w0, wg0i = (int)wg0;
  const int Li = L < 0x7fffffff ? (int)L : 0x7fffffff;
  auto tok = [&](int it) { return w0i + it * kDecWaves * kTile + col; };
  // fp8: load v of lane l is 16 bytes (chunk l & 7) of the tile's row
  // 8v + (l >> 3), so every load instruction reads 8 whole rows (1 KB), which
  // lets it stream with the non-temporal hint; bf16: lane (col, g) reads its
  // own half row.  Rows past L repeat row L-1 (bf16) or read as zeros (fp8);
  // their scores are dropped.
  auto load_tile = [&](i32x4 (&raw)[NV], float& sc, int it) {
    if constexpr (FP8) {
      // The tile's keys as a buffer resource (wave-uniform, built on the
      // scalar unit) that ends at the request's end: rows past it read as
      // zeros without touching memory (their scores are dropped).  Row
      // 8v + (lane >> 3) of the tile, chunk lane & 7, is byte 1024 v + 16 lane,
      // so the lane offsets are constants.  (The scale stays a clamped global
      // load: as a buffer load this compiler drains every load in flight at
      // the top of the unrolled loop.)
      const int t0 = w0i + it * kDecWaves * kTile;
      const int left = Li - t0;  // > 0: the tile index is clamped to the wave's last tile
      const __amdgpu_buffer_rsrc_t krs = buf_rsrc(kbase + (int64_t)t0 * kRowBytes, (uint32_t)left * kRowBytes);
#pragma unroll
      for (int v = 0; v < NV; ++v) raw[v] = buf_ld16_stream(krs, 16 * lane + 1024 * v);
      const int ss = t0 + col < Li ? t0 + col : Li - 1;
      sc = k_scale ? k_scale[off + ss] : 1.0f;
    } else {
      const int64_t t0 = w0 + (int64_t)it * kDecWaves * kTile;
      int64_t r = t0 + col;
      r = r < L ? r : L - 1;
      const uint8_t* p = kbase + r * kRowBytes;
#pragma unroll
      for (int v = 0; v < NV; ++v) raw[v] = ld16(p + 16 * v);
      sc = k_scale ? k_scale[off + r] : 1.0f;
    }
  };
  // The fp8 tile through this wave's LDS slice: 16-byte chunk c of row r
  // sits at chunk c ^ swz(r) of the row, so that both the row-wise writes
  // (8 lanes per row) and the key-wise reads (one row per lane) spread over
  // all banks, for 32 and for 64 banks of 4 bytes.  The wave's LDS
  // operations run in order, so the next tile's writes cannot overtake these
  // reads and no barrier is needed.
  auto swz = [](int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); };
  auto transpose = [&](const i32x4 (&raw)[NV], i32x4 (&kr)[NV]) {
    uint8_t* tl = ktl[FP8 ? wave : 0];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int r = 8 * v + (lane >> 3);
      *reinterpret_cast<i32x4*>(tl + r * 128 + (((lane & 7) ^ swz(r)) << 4)) = raw[v];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      kr[j] = *reinterpret_cast<const i32x4*>(tl + col * 128 + ((((g << 2) + j) ^ swz(col)) << 4));
  };
  // `it` is already clamped to a valid tile; `live` is false for the repeated
  // last tile that pads the pipeline, whose (identical) scores are not counted.
  auto compute = [&](const i32x4 (&raw)[NV], float sc, int it, bool live) {
    i32x4 kr[FP8 ? NV : 1];
    if constexpr (FP8) transpose(raw, kr);
    f32x16 a0 = {}, a1 = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 kb;
      if constexpr (FP8) {
        const i32x4 v = kr[j >> 1];
        kb = (j & 1) ? fp8x8_to_bf16x8(v.z, v.w) : fp8x8_to_bf16x8(v.x, v.y);
      } else {
        kb = __builtin_bit_cast(bf16x8, raw[j]);
      }
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][j], kb, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][j], kb, a1, 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(wl[0][r], relu(a0[r]), part);
      part = fmaf(wl[1][r], relu(a1[r]), part);
    }
    part = sum_halves(part);
    // LDS only from here on (no global-memory op under a branch, so the
    // loads' wait counting stays exact).  Positions past L are dropped at the
    // final write; a repeated padding tile rewrites identical values.
    const int s = tok(it);
    const uint32_t key = score_key(part * sc);
    if (g == 0) ssc[s - wg0i] = key;
    if (select && live && g == 0 && s < Li) atomicAdd(&lhist[key >> kSelShift], 1u);
  };

  if (nt > 0) {
    // A ring of kStages tile buffers: while tile it is computed, the loads of
    // tiles it+1 .. it+kStages-1 are in flight, the last of them issued just
    // before the compute.  Tile indices past nt-1 repeat the last tile.
    i32x4 buf[kStages][NV];
    float scb[kStages];
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) load_tile(buf[st], scb[st], st < nt ? st : nt - 1);
    const int nit = (nt + kStages - 1) / kStages * kStages;
    for (int base = 0; base < nit; base += kStages) {
      set_progress_priority(base, nit);
#pragma unroll
      for (int st = 0; st < kStages; ++st) {
        const int it = base + st;
        const int nx = it + kStages - 1;
        load_tile(buf[(st + kStages - 1) % kStages], scb[(st + kStages - 1) % kStages], nx < nt ? nx : nt - 1);
        compute(buf[st], scb[st], it < nt ? it : nt - 1, it < nt);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();
  // Scores of positions wg0 .. min(wg0 + chunk, L) - 1, 16 bytes per store
  // where the request's offset keeps them aligned (bucket mode: only when the
  // caller asked for them).
  const int64_t n = (L - wg0) < chunk ? (L - wg0) : chunk;
  if (scores) {
    float* dst = scores + off + wg0;
    if (((off + wg0) & 3) == 0) {
      const int64_t n4 = n >> 2;
      for (int64_t i = tid; i < n4; i += 256) {
        const i32x4 kv = *reinterpret_cast<const i32x4*>(&ssc[4 * i]);
        *reinterpret_cast<f32x4*>(dst + 4 * i) =
            f32x4{key_score(kv.x), key_score(kv.y), key_score(kv.z), key_score(kv.w)};
      }
      for (int64_t i = 4 * n4 + tid; i < n; i += 256) dst[i] = key_score(ssc[i]);
    } else {
      for (int64_t i = tid; i < n; i += 256) dst[i] = key_score(ssc[i]);
    }
  }
  if (!select) return;

  // This workgroup's share of the request's level-0 histogram, as 16-bit
  // partials (a workgroup covers at most 8192 positions); in bucket mode as
  // prefix counts, with its candidate list.
  const int64_t pi = (int64_t)b * sel.nwg + blockIdx.x;
  if (sel.bucket)
    bucket_epilogue<256, kDecMaxChunk>(lhist, ssc, (int)n, k, (uint32_t)wg0, sel.part + pi * kSelBins,
                                       sel.blist + pi * sel.chunk, wsum, sh_floor);
  else
    store_partial<256>(lhist, sel.part + pi * kSelBins, sel.cpart + pi * kSelCoarse);
}

}  // namespace

int64_t decode_chunk(int64_t n_tok, int32_t B) {
  // Tiles per wave: about two workgroups per CU when there is enough work (the
  // kernel holds two 4-wave workgroups per CU), long runs so each workgroup's
  // one-off query load, histogram store and list epilogue are amortised.
  int64_t tpw = n_tok / ((int64_t)512 * kDecWaves * kTile);
  // Smaller batches (e.g. ragged requests of 8K-32K): there a workgroup's
  // fixed costs (query load, list epilogue, and its partial and list in the
  // selection's reads) outweigh its streaming, and each request can add a
  // partly filled last workgroup.  They take about one workgroup per CU,
  // n_tok / chunk + B <= 256, up to 4096 positions per workgroup (which every
  // k can select from in bucket mode).  On the B = 32 ragged 8K-32K batch this
  // measured 39 -> 32 us for the scan and 12.3 -> 9.4 us for the top-k against
  // 1280-position workgroups.
  if (tpw < 16) {
    const int64_t room = 256 - (B < 128 ? (int64_t)B : 128);
    const int64_t fit = (n_tok + room * kDecWaves * kTile - 1) / (room * kDecWaves * kTile);
    tpw = fit > tpw ? (fit < 32 ? fit : 32) : tpw;
  }
  tpw = tpw < 4 ? 4 : (tpw > kDecMaxTpw ? kDecMaxTpw : tpw);
  return (int64_t)kDecWaves * tpw * kTile;
}

hipError_t launch_decode_score(const uint16_t* q, const float* w, const void* kc, bool kc_fp8,
                               const float* k_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t H, int32_t k,
                               float* scores, const SelWs& sel, hipStream_t stream) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  const int64_t chunk = decode_chunk(n_tok, B);
  const int tpw = (int)(chunk / ((int64_t)kDecWaves * kTile));
  dim3 grid((unsigned)((max_len + chunk - 1) / chunk), (unsigned)B);
  dim3 block(64 * kDecWaves);
  if (kc_fp8)
    return launch_kernel(decode_score_kernel<true>, grid, block, 0, stream, q, w, (const uint8_t*)kc, k_scale,
                         kv_off, H, tpw, k, scores, sel);
  return launch_kernel(decode_score_kernel<false>, grid, block, 0, stream, q, w, (const uint8_t*)kc, k_scale,
                       kv_off, H, tpw, k, scores, sel);
}

}  // namespace li
