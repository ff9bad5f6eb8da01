// Prefill scan of the lightning indexer on gfx950: T new query tokens of one
// sequence against its L-token key cache, causal.
//
//   S[t][s] = q_scale[t] * k_scale[s] * sum_h w[t][h] * ReLU(q_hat[t][h] . k_hat[s]),
//   visible iff s <= qpos0 + t
//
// This is a dense contraction (M = T*64 query-head rows, N = L keys, K = 128)
// with fp8 operands, so it runs on the fp8 matrix cores
// (v_mfma_f32_16x16x128_f8f6f4, OCP E4M3 for both operands); fully masked key
// tiles are never computed.
//
// The epilogue is the expensive part: every (head, key) product needs a ReLU
// and a weighted add, which on the vector ALU costs as much time as the MFMA
// that produced it.  It is halved with the identity
//   sum_h w_h ReLU(x_h) = 1/2 * ( sum_h w_h |x_h|  +  sum_h w_h x_h ):
// the first sum is one FMA per element (|x| is a free source modifier), and
// the second is linear in the key,
//   sum_h w_h x_h = u . k_hat,   u = sum_h w_h q_hat_h,
// so it runs on the matrix cores as a few extra MFMA rows.  u is stored as
// four fp8 rows f_i with power-of-two scales, u ~= sum_i 2^e_i f_i, each row
// encoding what the previous rows left over (relative residual ~2^-16; the
// tolerance on a score is 2e-3 of sum_h |w_h x_h|).
//
// Mapping: a wave owns two query tokens: four 16-row blocks of heads per
// token plus one block holding both tokens' u rows (rows 4*slot + i), all in
// registers, and walks the visible keys 32 at a time as two 16-key blocks, one
// 16x16x128 product per (head block, key block) covering all 128 dims.  Small
// products keep the epilogue's registers small, so each block's epilogue runs
// on the VALU while the matrix core works on the products issued after it
// (two blocks ahead).  A lane's block results are 4 heads of one key; after
// the tile, two permlane32 swaps and one permlane16 swap fold the four lane
// groups' head sums so that lane l holds token slot l >> 5 at key l & 31.
//
// A wave owns whole rows, so it also builds each row's level-0 selection
// histogram in LDS and finds the row's threshold bin for the top-k itself.
//
// Candidates instead of a dense score matrix: a row's final top-k threshold is
// at least the k-th largest key seen so far, so a key whose level-0 bin is
// below the bin of that running k-th largest can never be selected.  Each row
// keeps such a floor (recomputed from its LDS histogram whenever k more keys
// have passed it) and appends the (key, position) pairs at or above it, in
// position order, to its own candidate list; on N(0,1)-like rows of 65536 keys
// at k = 2048 that is about a sixth of the row.  The dense scores are written
// only when the caller asks for them.
#include "li_device.h"
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfTokPerWave = 2;
constexpr int kPfTokPerBlock = kPfWaves * kPfTokPerWave;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ i32x8 ld32(const uint8_t* p) {
  const i32x4 x = ld16(p), y = ld16(p + 16);
  i32x8 r = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
  return r;
}

// Row histograms are packed two 16-bit bins per 32-bit word (bin b in the
// half b & 1 of word b >> 1) to halve their LDS footprint.  A bin that passes
// 65535 carries into its neighbour or wraps, so the bins then no longer sum to
// the row's visible count; that is detected here and the row is marked for
// the top-k kernel to rebuild its histogram itself (thr[3] = 0).

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

// Where the kk-th largest key of a row falls in its histogram: the bin, the
// keys in bins above it and in it.  found is false when the row holds fewer
// than kk keys; ok is false when the bins do not sum to the row's count.
struct Cross {
  uint32_t bin, above, eq;
  bool found, ok;
};

// Both rows of a wave at once: lane half g takes the histogram of row slot g
// (packed words hist[g * kSelBins / 2 ...]) holding `counted` keys.  Lane c of
// the half sums bins [64c, 64c + 64) with eight 16-byte reads; a suffix sum
// over the half finds the lane whose bins hold the crossing, then each lane
// reads one word (two bins) of that lane's range and a second suffix sum finds
// the bin.  Every lane of the half returns its row's result.
__device__ Cross pair_cross(const uint32_t* hist, uint32_t kk, uint32_t counted) {
  const int lane = threadIdx.x & 63, c = lane & 31, g = lane >> 5;
  const uint32_t* h = hist + (kSelBins / 2) * g;
  const i32x4* p = reinterpret_cast<const i32x4*>(h + 32 * c);
  i32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = p[j];
  const u16x2 ones = {1, 1};
  auto add2 = [&](int w, uint32_t acc) { return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, w), ones, acc, false); };
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s = add2(v[j].x, add2(v[j].y, add2(v[j].z, add2(v[j].w, s))));
  // keys in the bins of lanes >= c of the half
  auto suffix = [&](uint32_t x) {
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_down((int)x, d, 32);
      x += c + d < 32 ? o : 0u;
    }
    return x;
  };
  const uint32_t suf = suffix(s);
  Cross r;
  r.ok = (uint32_t)__shfl((int)suf, 0, 32) == counted;
  const uint64_t m1 = __builtin_amdgcn_ballot_w64(suf - s < kk && suf >= kk);
  const uint32_t h1 = (uint32_t)(m1 >> (32 * g));
  r.found = h1 != 0u;
  const int c1 = r.found ? __builtin_ctz(h1) : 0;
  const uint32_t above1 = (uint32_t)__shfl((int)(suf - s), c1, 32);
  const uint32_t w = h[32 * c1 + c];
  const uint32_t lo = w & 0xFFFFu, hi = w >> 16, cnt = lo + hi;
  const uint32_t suf2 = suffix(cnt) + above1;
  const uint64_t m2 = __builtin_amdgcn_ballot_w64(suf2 - cnt < kk && suf2 >= kk);
  const uint32_t h2 = (uint32_t)(m2 >> (32 * g));
  const int c2 = h2 ? __builtin_ctz(h2) : 0;
  // in lane c2: the upper bin of its word first
  const uint32_t ab = suf2 - cnt;
  const bool upper = ab + hi >= kk;
  const uint32_t bin = (uint32_t)(64 * c1 + 2 * c) + (upper ? 1u : 0u);
  r.bin = (uint32_t)__shfl((int)bin, c2, 32);
  r.above = (uint32_t)__shfl((int)(upper ? ab : ab + hi), c2, 32);
  r.eq = (uint32_t)__shfl((int)(upper ? hi : lo), c2, 32);
  r.found = r.found && h2 != 0u;
  return r;
}

constexpr int kLinTerms = kLinRows;  // fp8 rows per token for u
constexpr int kPfRing = 4;   // LDS key-tile slots per workgroup
constexpr int kPfLead = 5;   // a tile's global loads are issued this many tiles before it is computed
constexpr int kPfWrite = 2;  // ... and written to LDS this many tiles before
constexpr int kPfRegs = kPfLead - kPfWrite + 1;  // register slots for loads in flight
static_assert(kPfRegs == 4 && kPfRing == 4, "the main loop is unrolled by 4");
constexpr int kTileBytes = 32 * 128;
constexpr int kFloorGrowShift = 1;

// u[t][d] = sum_h w[t][h] * q_hat[t][h][d] in fp32, then split into
// kLinTerms fp8 rows: row i holds round(r_i * 2^-e_i) with 2^e_i chosen so the
// largest |r_i| lands in [128, 256), and r_{i+1} = r_i - 2^e_i * row_i (the
// residual uses the row's exact fp8 value, so any rounding of the encoder is
// compensated by the next row).  Two tokens per 256-thread block, one dim per
// thread.
__global__ __launch_bounds__(256) void prefill_linear_kernel(const uint8_t* __restrict__ q,
                                                             const float* __restrict__ w, int T, int H,
                                                             uint8_t* __restrict__ uq,
                                                             float* __restrict__ usc) {
  __shared__ float red[4];
  const int slot = threadIdx.x >> 7, d = threadIdx.x & 127;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 2 + slot;
  const int tt = t < T ? t : T - 1;
  // All of a thread's loads are issued before the arithmetic (clamped head
  // index, zero weight past H), 16 heads per batch.
  float u = 0.0f;
  for (int h0 = 0; h0 < H; h0 += 16) {
    uint32_t qb[16];
    float wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = h0 + i < H ? h0 + i : H - 1;
      qb[i] = q[((int64_t)tt * H + h) * 128 + d];
      wv[i] = w[(int64_t)tt * H + h];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) u = fmaf(h0 + i < H ? wv[i] : 0.0f, fp8_to_f32(qb[i]), u);
  }
  float r = u;
#pragma unroll
  for (int i = 0; i < kLinTerms; ++i) {
    const float m = wave_max(fabsf(r));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float mt = fmaxf(red[2 * slot], red[2 * slot + 1]);
    __syncthreads();
    // exponent of the row scale; a (near-)zero residual gets an all-zero row
    const int e = mt > 0x1p-100f ? ilogbf(mt) - 7 : 0;
    const float sc = ldexpf(1.0f, e);
    uint32_t f = 0u;
    if (mt > 0x1p-100f) {
      const float v = r * ldexpf(1.0f, -e);  // |v| < 256: no saturation
      f = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
    }
    r -= fp8_to_f32(f) * sc;
    if (t < T) {
      uq[((int64_t)t * kLinTerms + i) * 128 + d] = (uint8_t)f;
      if (d == 0) usc[(int64_t)t * kLinTerms + i] = sc;
    }
  }
}

// DENSE: also write every score (out_scores given).  clist [T][L] (key,
// position) pairs and ccnt [T] receive each row's candidate list.
template <bool KSCALE, bool DENSE>
__global__ __launch_bounds__(256) void prefill_score_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ uq, const float* __restrict__ usc, const uint8_t* __restrict__ kc,
    const float* __restrict__ k_scale, int T, int L, int qpos0, int H, int k, int fill_masked,
    float* __restrict__ scores, uint32_t* __restrict__ thr, uint2* __restrict__ clist, uint32_t* __restrict__ ccnt) {
  static_assert(kPfTokPerWave == 2 && kPfWaves == 4, "lane half g finishes token slot g; 4 loader waves");
  __shared__ __attribute__((aligned(16))) uint32_t phist[kPfWaves][kPfTokPerWave][kSelBins / 2];
  // Key tiles shared by the workgroup's waves (which walk the same keys): 32
  // keys x 128 bytes per slot, 16-byte chunk c of key r stored at chunk
  // c ^ (r & 7) so that the MFMA operand reads are free of bank conflicts.
  __shared__ __attribute__((aligned(16))) uint8_t ktile[kPfRing][kTileBytes];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col = lane & 31, g = lane >> 5;
  const int t_base = (blockIdx.x * kPfWaves + wave) * kPfTokPerWave;
  const int nt = t_base >= T ? 0 : ((T - t_base) < kPfTokPerWave ? (T - t_base) : kPfTokPerWave);
  // Token slot tk computes row trow[tk]; slots past the end of the chunk
  // repeat a valid token (so their stores rewrite identical values) and are
  // never counted in a histogram.
  int trow[kPfTokPerWave];
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk) trow[tk] = nt > 0 ? t_base + (tk < nt ? tk : 0) : T - 1;

  for (int i = lane; i < kPfTokPerWave * kSelBins / 2; i += 64) (&phist[wave][0][0])[i] = 0;

  // Query heads (A operand: row = head 16*hb + c16, dims 32*g4 .. +31), the
  // weights of the heads whose results this lane holds (rows 4*g4 + i of each
  // head block), and the u rows: A row c16 < 8 is u row (c16 & 3) of token
  // slot c16 >> 2.  Lane group g4 < 2 holds token slot g4's u results and its
  // u-row scales; the other groups' rows are zero.
  const int c16 = lane & 15, g4 = lane >> 4;
  i32x8 qa[kPfTokPerWave][4];
  float wl[kPfTokPerWave][4][4];
#pragma unroll
  for (int tk = 0; tk < kPfTokPerWave; ++tk) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int head = 16 * hb + c16;
      // Clamped, unconditional load (rows past H are zeroed afterwards).
      i32x8 v = ld32(q + ((int64_t)trow[tk] * H + (head < H ? head : H - 1)) * 128 + 32 * g4);
      if (head >= H) v = i32x8{};
      qa[tk][hb] = v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hr = 16 * hb + 4 * g4 + i;
        const float wv = w[(int64_t)trow[tk] * H + (hr < H ? hr : H - 1)];
        wl[tk][hb][i] = hr < H ? wv : 0.0f;
      }
    }
  }
  i32x8 ua;
  {
    const bool urow = c16 < kLinTerms * kPfTokPerWave;
    const int uc = urow ? c16 : 0;
    i32x8 v = ld32(uq + ((int64_t)trow[uc >> 2] * kLinTerms + (uc & 3)) * 128 + 32 * g4);
    if (!urow) v = i32x8{};
    ua = v;
  }
  float us[kLinTerms];
  {
    const int ut = trow[g4 < kPfTokPerWave ? g4 : 0];
#pragma unroll
    for (int i = 0; i < kLinTerms; ++i) {
      const float v = usc[(int64_t)ut * kLinTerms + i];
      us[i] = g4 < kPfTokPerWave ? v : 0.0f;
    }
  }
  // This half's token (the one lane l finishes: slot l >> 5) and its scale.
  const int tg = trow[g];
  const float sq = (q_scale ? q_scale[tg] : 1.0f) * 0.5f;
  // The last key position this lane's row counts (-1 for a slot past the end
  // of the chunk): visible keys inside the cache.
  const int last_counted = g < nt ? min(qpos0 + tg, L - 1) : -1;

  // Tiles this wave needs, and tiles the workgroup walks (every wave takes
  // part in every tile's barrier; the extra tiles are fully masked for it).
  const int wg_t_end = (blockIdx.x + 1) * kPfTokPerBlock < T ? (blockIdx.x + 1) * kPfTokPerBlock : T;
  const int n_tiles = nt > 0 ? (qpos0 + t_base + nt + 31) / 32 : 0;
  const int n_wg = (qpos0 + wg_t_end + 31) / 32;
  auto clamp_tile = [&](int it) { return it < n_wg ? it : n_wg - 1; };
  // Key row of tile `it` for this lane, clamped into the cache: a lane past
  // the end recomputes row L-1 and rewrites that row's own score.
  auto key_row = [&](int it) {
    const int s = it * 32 + col;
    return s < L ? s : L - 1;
  };
  // This wave's share of a tile: keys 8*wave + lane/8, chunk lane % 8.
  const int ld_key = 8 * wave + (lane >> 3), ld_chunk = lane & 7;
  const int ld_off = ld_key * 128 + 16 * (ld_chunk ^ ((ld_key >> 1) & 7));
  auto gload = [&](int it) {
    int row = it * 32 + ld_key;
    row = row < L ? row : L - 1;
    return ld16(kc + (int64_t)row * 128 + 16 * ld_chunk);
  };
  auto lds_put = [&](int slot, i32x4 v) { *reinterpret_cast<i32x4*>(&ktile[slot][ld_off]) = v; };
  // B operand of key block j: key 16*j + c16, dims 32*g4 .. +31 (chunks 2*g4
  // and 2*g4 + 1).  Each 16-lane group of a 16-byte read then touches 16
  // different 4-bank groups (key parity x swizzled chunk), so the reads are
  // free of bank conflicts, and so are the writes (two keys x eight chunks).
  auto lds_get = [&](int slot, i32x8 (&kb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = 16 * j + c16, f = (key >> 1) & 7;
      const uint8_t* base = &ktile[slot][key * 128];
      const i32x4 x = *reinterpret_cast<const i32x4*>(base + 16 * ((2 * g4) ^ f));
      const i32x4 y = *reinterpret_cast<const i32x4*>(base + 16 * ((2 * g4 + 1) ^ f));
      kb[j] = i32x8{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    }
  };
  auto load_scale = [&](int it) {
    if constexpr (KSCALE) return k_scale[key_row(it)];
    else return 1.0f;
  };

  // Candidate list state: per row slot, the number of pairs appended (nc0,
  // nc1, wave-uniform); the floor bin of the lane's own row.
  uint32_t floor_bin = 0u, nc0 = 0u, nc1 = 0u;
  // The wave's candidate rows as one buffer resource (L <= kPrefillMaxL keeps
  // it under 1 GiB).  A lane with nothing to append stores at an offset past
  // its end, which the hardware drops: the store is straight-line code in
  // every tile, so the waits for the key loads in flight stay exact.
  const uint32_t row_bytes = (uint32_t)L * 8u;
  const __amdgpu_buffer_rsrc_t lrsrc = __builtin_amdgcn_make_buffer_rsrc(
      clist + (int64_t)(nt > 0 ? t_base : 0) * L, (short)0, (int)(row_bytes * (uint32_t)nt), kBufferWord3);
  const uint32_t row_off = (uint32_t)g * row_bytes;
  auto compute = [&](const i32x8 (&kb)[2], float sk, int it, bool live) {
    const int s = it * 32 + col;
    const int srow = key_row(it);
    __builtin_amdgcn_s_setprio(1);
    // 18 products per tile: for key block j, the four head blocks of token
    // slot 0, those of slot 1, then the u block.  Product n + 2 is issued
    // before the epilogue of product n; the scheduling barriers keep that
    // order (the compiler would otherwise group the products together).
    constexpr int kBlk = 2 * (4 * kPfTokPerWave + 1);
    float P[kPfTokPerWave][2] = {};
    float lsum[2] = {};
    f32x4 acc[kBlk];
    auto issue = [&](int n) {
      const int j = n / 9, m = n % 9;
      const f32x4 z = {};
      acc[n] = m < 8 ? mfma_fp8_16(qa[m >> 2][m & 3], kb[j], z) : mfma_fp8_16(ua, kb[j], z);
    };
    auto epilogue = [&](int n) {
      const int j = n / 9, m = n % 9;
      if (m < 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) P[m >> 2][j] = fmaf(wl[m >> 2][m & 3][i], fabsf(acc[n][i]), P[m >> 2][j]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[j] = fmaf(us[i], acc[n][i], lsum[j]);
      }
    };
    issue(0);
    issue(1);
#pragma unroll
    for (int n = 0; n < kBlk; ++n) {
      if (n + 2 < kBlk) issue(n + 2);
      __builtin_amdgcn_sched_barrier(0);
      epilogue(n);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // u . k joins the token its rows belong to (lane group g4 holds slot g4's),
    // then the four lane groups' head sums fold onto lane l = (slot, key):
    // the 32-lane swap pairs groups {0,2} and {1,3} per slot, the 16-lane swap
    // pairs the key blocks.
    float R[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      R[j] = swap_sum32(P[0][j] + (g4 == 0 ? lsum[j] : 0.0f), P[1][j] + (g4 == 1 ? lsum[j] : 0.0f));
    const float pa = swap_sum16(R[0], R[1]);
    const bool vis = srow <= qpos0 + tg;
    const float val = vis ? pa * sq * sk : -INFINITY;
    // Straight-line store (a lane past the end rewrites row L-1 with its own
    // value) so the loads of the next tiles stay in flight.
    if constexpr (DENSE) scores[(int64_t)tg * L + srow] = val;
    // Unconditional LDS update (adds 0 where the score is not counted), so
    // the tile stays one basic block.
    const uint32_t key = score_key(val), b = key >> kSelShift;
    const bool counted = (live & (it < n_tiles)) & (s <= last_counted);
    atomicAdd(&phist[wave][g][b >> 1], (counted ? 1u : 0u) << (16 * (b & 1)));
    // Append the keys at or above the floor, ranked within the half by the
    // ballot (ascending key position = lane order).  The upper half's rank
    // counts the lower half's kept lanes too; its base takes them off.
    const bool keep = counted && b >= floor_bin;
    const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
    const uint32_t klo = (uint32_t)km, khi = (uint32_t)(km >> 32);
    const uint32_t clo = (uint32_t)__builtin_popcount(klo), chi = (uint32_t)__builtin_popcount(khi);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi(khi, __builtin_amdgcn_mbcnt_lo(klo, 0u));
    const uint32_t off = keep ? row_off + 8u * (rank + (g ? nc1 - clo : nc0)) : kBufferDrop;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{key, (uint32_t)srow}, lrsrc, off, 0, 0);
    nc0 += clo;
    nc1 += chi;
  };
  // Rows' floors move up on a schedule shared by the workgroup's waves (they
  // meet at a barrier every tile, so a refresh in one wave would stall the
  // others; refreshing together overlaps them): first once k keys have been
  // seen, then each time the keys seen grow by a factor 1 + 2^-kFloorGrowShift.
  // After step i, the keys counted for a row are its visible keys among the
  // first min(i, n_wg - 1) + 1 tiles.
  int next_refresh = k;
  auto refresh_floor = [&](int i) {
    const int seen = ((i < n_wg ? i : n_wg - 1) + 1) * 32;
    if (seen < next_refresh) return;  // uniform over the workgroup
    next_refresh = seen + max(seen >> kFloorGrowShift, 128);
    const int v = qpos0 + tg + 1;
    const Cross cr = pair_cross(&phist[wave][0][0], (uint32_t)k, g < nt ? (uint32_t)min(seen, min(L, v)) : 0u);
    floor_bin = cr.ok && cr.found ? cr.bin : 0u;
  };

  // Software pipeline over the workgroup's tiles (step i computes tile i):
  //   tile i+kPfLead: global -> registers (slot (i+kPfLead) % 4)
  //   tile i+kPfWrite: registers -> LDS slot (i+kPfWrite) % 4
  //   barrier; tile i: LDS -> MFMA operand, compute.
  // LDS slot (i+2)%4 last held tile i-2, which every wave finished before the
  // barrier of step i-1; tile i was written at step i-2, before two barriers.
  // The key scales ride in a register ring loaded kPfRegs steps ahead.
  i32x4 kreg[kPfRegs];
  float skr[kPfRegs];
  lds_put(0, gload(clamp_tile(0)));
  lds_put(1, gload(clamp_tile(1)));
#pragma unroll
  for (int j = kPfWrite; j <= kPfLead; ++j) kreg[j % kPfRegs] = gload(clamp_tile(j));
#pragma unroll
  for (int j = 0; j < kPfRegs; ++j) skr[j] = load_scale(clamp_tile(j));
  // The MFMA operand of tile i+1 is read from LDS while tile i is computed
  // (tile i+1 was written at step i-1, before the barrier of step i).
  i32x8 kbuf[2][2];
  const int nsteps = (n_wg + kPfRegs - 1) / kPfRegs * kPfRegs;
  __syncthreads();
  lds_get(0, kbuf[0]);
  for (int base = 0; base < nsteps; base += kPfRegs) {
#pragma unroll
    for (int st = 0; st < kPfRegs; ++st) {
      const int i = base + st;
      lds_put((st + kPfWrite) % kPfRing, kreg[(st + kPfWrite) % kPfRegs]);
      kreg[(st + kPfLead) % kPfRegs] = gload(clamp_tile(i + kPfLead));
      __syncthreads();
      lds_get((st + 1) % kPfRing, kbuf[(st + 1) & 1]);
      const int it = clamp_tile(i);
      compute(kbuf[st & 1], skr[st], it, i < n_wg);
      skr[st] = load_scale(clamp_tile(i + kPfRegs));
    }
    // Once per unrolled iteration, so that its four steps stay one block of
    // straight-line code for the scheduler.
    refresh_floor(base + kPfRegs - 1);
  }
  // Each row's list length (lane 0 of its half).
  if (col == 0 && g < nt) ccnt[tg] = g ? nc1 : nc0;
  __syncthreads();
  {
    // Each row's threshold bin (rows with more than k visible keys), or the
    // overflow mark.
    const int vis = qpos0 + tg + 1;
    const uint32_t n = (uint32_t)(vis < L ? vis : L);
    const Cross cr = pair_cross(&phist[wave][0][0], (uint32_t)k, g < nt ? n : 0u);
    if (col == 0 && g < nt && vis > k) {
      uint32_t* t = thr + (int64_t)tg * 4;
      if (cr.ok && cr.found) {
        t[0] = cr.bin;
        t[1] = cr.above;
        t[2] = cr.eq;
        t[3] = 1u;
      } else {
        t[3] = 0u;
      }
    }
  }
  if (DENSE && fill_masked) {
    for (int tk = 0; tk < nt; ++tk) {
      const int t = t_base + tk;
      for (int s = n_wg * 32 + lane; s < L; s += 64) scores[(int64_t)t * L + s] = -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_prefill_linear(const uint8_t* q, const float* w, int32_t T, int32_t H, uint8_t* uq,
                                 float* usc, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  return launch_kernel(prefill_linear_kernel, dim3((unsigned)((T + 1) / 2)), dim3(256), 0, stream, q, w, T, H, uq,
                       usc);
}

hipError_t launch_prefill_score(const uint8_t* q, const float* q_scale, const float* w,
                                const uint8_t* uq, const float* usc, const uint8_t* kc,
                                const float* k_scale, int32_t T, int32_t L, int32_t qpos0, int32_t H,
                                int32_t k, float* scores, const SelWs& sel, uint2* clist, uint32_t* ccnt,
                                hipStream_t stream) {
  if (T <= 0 || L <= 0) return hipSuccess;
  dim3 grid((unsigned)((T + kPfTokPerBlock - 1) / kPfTokPerBlock));
  const int fill = scores ? 1 : 0;
  const dim3 block(64 * kPfWaves);
  if (k_scale) {
    if (scores)
      return launch_kernel(prefill_score_kernel<true, true>, grid, block, 0, stream, q, q_scale, w, uq, usc, kc,
                           k_scale, T, L, qpos0, H, k, fill, scores, sel.thr, clist, ccnt);
    return launch_kernel(prefill_score_kernel<true, false>, grid, block, 0, stream, q, q_scale, w, uq, usc, kc,
                         k_scale, T, L, qpos0, H, k, fill, scores, sel.thr, clist, ccnt);
  }
  if (scores)
    return launch_kernel(prefill_score_kernel<false, true>, grid, block, 0, stream, q, q_scale, w, uq, usc, kc,
                         k_scale, T, L, qpos0, H, k, fill, scores, sel.thr, clist, ccnt);
  return launch_kernel(prefill_score_kernel<false, false>, grid, block, 0, stream, q, q_scale, w, uq, usc, kc,
                       k_scale, T, L, qpos0, H, k, fill, scores, sel.thr, clist, ccnt);
}

}  // namespace li
