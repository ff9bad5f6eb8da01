// Per-row top-k selection on gfx950 (the step that turns indexer scores into
// the index tensor: "IndexCache: Cross-Layer Index Reuse for Sparse
// Attention", Deep Dive, the F layer takes top-k of its scores).
//
// Scores map to order-preserving uint32 keys (-0 folded onto +0).  The
// selection is a radix select whose first level is the top 11 key bits: the
// threshold bin b* is the level-0 bin that holds the k-th largest key.  Then
// the keys whose bin is >= b* -- at most (k-1) + |b*| of them -- are gathered
// in position order (into registers or LDS), two more histogram levels over
// the keys of bin b* give the exact k-th key T and the number m of keys equal
// to T that still fit, and an ordered compaction writes the kept positions:
//   slot = #greater-before + min(#equal-before, m),
// so the output is in ascending position order and the lower position wins a
// tie.  Rows with at most k visible keys return all of them; unused slots are
// -1.  Candidate sets too large for registers and LDS (heavy ties) are
// resolved the same way from global memory.  Integer histograms make every
// path deterministic.
//
// Two kernels:
//   segmented (decode, LatentIndex: few long rows): one workgroup per
//     (8192-score segment, row).  Each sums the row's per-scan-workgroup
//     partial histograms to find b*, keeps its segment's candidates, and the
//     last workgroup of the row to finish (device-scope counter; the scan
//     kernel zeroes it) performs the final selection over all of them.  One
//     launch after the scan.
//   per-row (prefill, HS followers, standalone): one workgroup per row, which
//     builds or is handed the level-0 histogram, collects its own candidates
//     into LDS and finishes.
#include "li_internal.h"
#include "li_select.h"

namespace li {

// Phase stamps of the bucket top-k, a measurement aid compiled in only with
// -DLI_STAMPS (build.py --stamps, a separate library): thread 0 of the row's
// workgroup records the 100 MHz real-time counter after each phase's
// barrier.  The product build has none of this code.
#ifdef LI_STAMPS
constexpr int kStampRows = 64, kStampPhases = 10;
__device__ unsigned long long li_stamp_buf[kStampRows * kStampPhases];
#define LI_STAMP(i)                                                                              \
  do {                                                                                           \
    if (threadIdx.x == 0 && blockIdx.x < kStampRows)                                             \
      li_stamp_buf[blockIdx.x * kStampPhases + (i)] = __builtin_amdgcn_s_memrealtime();          \
  } while (0)
#else
#define LI_STAMP(i) \
  do {              \
  } while (0)
#endif
namespace {

constexpr int kRowThreads = 512;   // per-row kernel
constexpr int kSegThreads = 512;   // segmented kernel
constexpr int kMaxCap = 18432;     // largest LDS candidate buffer (pairs) of either kernel (144 KB)
constexpr int kRegCand = 16;       // segmented kernel: candidates per thread held in registers

struct Row {
  const float* p;
  int64_t n;
  const int32_t* map;  // position map (candidates) or null
  int32_t* out;
};

__device__ Row get_row(const TopkRows& a, int r, int32_t* sh) {
  Row row;
  row.map = nullptr;
  row.out = a.out + (int64_t)r * a.k;
  switch (a.mode) {
    case kRowsOffsets: {
      const int b = r / a.G, l = r - b * a.G;
      const int64_t off = a.kv_off[b];
      row.p = a.scores + (int64_t)l * a.row_stride + off;
      row.n = a.kv_off[b + 1] - off;
      break;
    }
    case kRowsCausal: {
      row.p = a.scores + (int64_t)r * a.row_stride;
      const int64_t vis = (int64_t)a.qpos0 + r + 1;
      row.n = vis < a.n ? vis : a.n;
      break;
    }
    case kRowsCands: {
      const int b = r / a.G;
      const int32_t* cand = a.cand + (int64_t)b * a.C;
      // Valid candidates come first (ascending), then -1 padding: find the first -1.
      if (threadIdx.x == 0) {
        int lo = 0, hi = a.C;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (cand[mid] < 0) hi = mid; else lo = mid + 1;
        }
        sh[0] = lo;
      }
      __syncthreads();
      row.p = a.scores + (int64_t)r * a.C;
      row.n = sh[0];
      row.map = cand;
      break;
    }
    default: {
      row.p = a.scores + (int64_t)r * a.row_stride;
      const int64_t len = a.row_len ? a.row_len[r] : a.n;
      row.n = len < a.row_stride ? len : a.row_stride;  // never read past the row
      break;
    }
  }
  if (row.n < 0) row.n = 0;
  return row;
}

__device__ __forceinline__ int32_t map_pos(const Row& row, int64_t i) {
  return row.map ? row.map[i] : (int32_t)i;
}

// out[slot[e]] = position src[e] (through the row's map when it has one) for
// the entries with 0 <= slot < kk.  The map loads are all issued before the
// first store: gfx9's vmcnt counts stores too, so a load issued between stores
// (or under a branch) would make every store wait for all earlier ones.
template <int E>
__device__ __forceinline__ void emit_slots(const Row& row, const int32_t (&slot)[E],
                                           const int32_t (&src)[E], int64_t kk) {
  if (row.map) {
    int32_t pv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) pv[e] = row.map[slot[e] >= 0 ? src[e] : 0];  // row.n >= 1 here
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (slot[e] >= 0 && slot[e] < kk) row.out[slot[e]] = pv[e];
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (slot[e] >= 0 && slot[e] < kk) row.out[slot[e]] = src[e];
  }
}

// Key of element i of p[0 .. n-1] (n >= 1), loaded without a branch: an index
// past the end reads element n-1 instead, and the caller ignores that key.
// (A load under a branch makes the compiler wait for it before the branch
// joins, which serialises a batch of loads.)
__device__ __forceinline__ uint32_t key_clamped(const float* p, int64_t i, int64_t n) {
  return score_key(p[i < n ? i : n - 1]);
}

// Writes all n visible positions and pads the row with -1 (rows with n <= k).
template <int NT>
__device__ void keep_all(const Row& row, int64_t n, int k) {
  for (int64_t i = threadIdx.x; i < k; i += NT) row.out[i] = (i < n) ? map_pos(row, i) : -1;
}

// Given per-thread counts of PER consecutive digits taken in descending order
// (thread t owns digits top - t*PER - i), find the digit holding the
// `remaining`-th largest key: {digit, #keys in higher digits, #keys in it}
// land in out[0..2].  Ends with a barrier.
template <int NT, int PER>
__device__ void find_digit(const uint32_t (&h)[PER], int top, uint32_t remaining, uint32_t* wsum,
                           uint32_t* out) {
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += h[i];
  uint32_t total;
  uint32_t run = block_excl_scan<NT>(sum, wsum, total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < remaining && run + h[i] >= remaining) {
      out[0] = (uint32_t)(top - ((int)threadIdx.x * PER + i));
      out[1] = run;
      out[2] = h[i];
    }
    run += h[i];
  }
  __syncthreads();
}

// The digit of an nb-bin histogram (nb = 2048 or 1024) that holds the
// `remaining`-th largest key; {digit, #keys above it, #in it} land in out[0..2].
template <int NT>
__device__ void hist_digit(const uint32_t* hist, int nb, uint32_t remaining, uint32_t* wsum,
                           uint32_t* out) {
  const int tid = threadIdx.x;
  constexpr int PER = kSelBins / NT;  // digits per thread when nb = 2048
  if (nb == kSelBins) {
    uint32_t h[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) h[i] = hist[nb - 1 - (tid * PER + i)];
    find_digit<NT, PER>(h, nb - 1, remaining, wsum, out);
  } else {  // nb = 1024
    constexpr int PH = PER / 2;
    uint32_t h[PH];
#pragma unroll
    for (int i = 0; i < PH; ++i) h[i] = hist[nb - 1 - (tid * PH + i)];
    find_digit<NT, PH>(h, nb - 1, remaining, wsum, out);
  }
}

// One radix level over `count` keys: histogram of the nb digits at `shift`
// among the keys matching (prefix, pmask), then the digit holding the
// `remaining`-th largest.  Leaves {digit, #keys above it, #in it} in out.
template <int NT, typename KeyAt>
__device__ void radix_level(KeyAt key_at, int64_t count, uint32_t prefix, uint32_t pmask, int shift,
                            int nb, uint32_t remaining, uint32_t* hist, uint32_t* wsum,
                            uint32_t* out) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kSelBins; i += NT) hist[i] = 0;
  __syncthreads();
  for (int64_t i = tid; i < count; i += NT) {
    const uint32_t key = key_at(i);
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
  }
  __syncthreads();
  hist_digit<NT>(hist, nb, remaining, wsum, out);
}

// Ordered compaction over `count` candidates in position order: keep keys > T
// and the first m keys equal to T, writing slot = #gt-before + min(#eq-before, m).
template <int NT, typename KeyAt, typename PosAt>
__device__ void compact(const Row& row, KeyAt key_at, PosAt pos_at, int64_t count, uint32_t T,
                        uint32_t m, int64_t kk, uint32_t* wsum) {
  const int tid = threadIdx.x;
  uint32_t gt_run = 0, eq_run = 0;
#pragma unroll 1
  for (int64_t base = 0; base < count; base += 4 * NT) {
    const int64_t i0 = base + 4 * tid;
    uint32_t fl[4];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e < count ? i0 + e : count - 1;  // clamped, branch-free read
      const uint32_t key = key_at(i);
      fl[e] = i0 + e < count ? (key > T ? 2u : (key == T ? 1u : 0u)) : 0u;
      cg += fl[e] >> 1;
      ce += fl[e] & 1u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<NT>((cg << 16) | ce, wsum, total);
    uint32_t gb = gt_run + (ex >> 16), eb = eq_run + (ex & 0xFFFFu);
    int32_t slot[4], src[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      slot[e] = -1;
      src[e] = 0;
      if (fl[e] == 2u) {
        slot[e] = (int32_t)(gb + (eb < m ? eb : m));
        ++gb;
      } else if (fl[e] == 1u) {
        if (eb < m) slot[e] = (int32_t)(gb + eb);
        ++eb;
      }
      if (slot[e] >= 0) src[e] = (int32_t)pos_at(i0 + e);
    }
    emit_slots<4>(row, slot, src, kk);
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
  }
}

// Radix levels first_level..2 (11/11/10 bits) over keys read through key_at,
// then the ordered compaction.  Used on LDS candidates (first_level = 1, the
// level-0 digit already known) and on whole rows in global memory (0).
template <int NT, typename KeyAt, typename PosAt>
__device__ void select_keys(const Row& row, KeyAt key_at, PosAt pos_at, int64_t count,
                            uint32_t prefix, uint32_t pmask, uint32_t remaining, int first_level,
                            int64_t kk, uint32_t* hist, uint32_t* wsum, uint32_t* out) {
#pragma unroll 1
  for (int level = first_level; level < 3; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int nb = level == 2 ? 1024 : 2048;
    radix_level<NT>(key_at, count, prefix, pmask, shift, nb, remaining, hist, wsum, out);
    prefix |= out[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    remaining -= out[1];
    __syncthreads();
  }
  compact<NT>(row, key_at, pos_at, count, prefix, remaining, kk, wsum);
}

// select_keys over candidates held in registers: thread t holds candidates
// t + NT*j (j < R), so (round j, wave, lane) is position order; entries at or
// past `count` are ignored.  The histograms are built from the registers, a
// level whose threshold digit is kept whole ends the descent (keys are then
// compared on the digits resolved so far), and the ordered compaction ranks
// each round with two ballots (greater / equal) plus one block-wide scan of
// the packed per-(round, wave) counts.  rcnt holds R * NT / 64 entries.
template <int NT, int R>
__device__ void select_regs(const Row& row, const uint2 (&v)[R], int64_t count, uint32_t prefix,
                            uint32_t pmask, uint32_t remaining, int64_t kk, uint32_t* hist,
                            uint32_t* wsum, uint32_t* rcnt, uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  constexpr int kW = NT / 64;
  static_assert(R * kW <= NT, "one (round, wave) count per thread");
  // Rounds past the last candidate hold nothing: skipped with a wave-uniform
  // branch (the finishing workgroup's time is VALU issue on 2 waves per SIMD,
  // and a 131072-score row at k = 2048 fills about 6 of 16 rounds).
  const int nr = (int)((count + NT - 1) / NT);
#pragma unroll 1
  for (int level = 1; level < 3; ++level) {
    const int shift = level == 1 ? 10 : 0;
    const int nb = level == 1 ? kSelBins : kSelBins / 2;
    for (int i = tid; i < kSelBins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j < nr) {
        if (j * NT + tid < (int)count && (v[j].x & pmask) == prefix)
          atomicAdd(&hist[(v[j].x >> shift) & (uint32_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    hist_digit<NT>(hist, nb, remaining, wsum, out);
    prefix |= out[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    remaining -= out[1];
    const bool whole = out[2] == remaining;
    __syncthreads();
    if (whole) break;
  }
  // Counts are < 2^16 (count <= R * NT), so (greater, equal) share one word.
  // The ballots are taken again in the write pass rather than kept.
  const int cnt32 = (int)count;
  auto gt = [&](int j) { return __ballot(j * NT + tid < cnt32 && (v[j].x & pmask) > prefix); };
  auto eq = [&](int j) { return __ballot(j * NT + tid < cnt32 && (v[j].x & pmask) == prefix); };
#pragma unroll
  for (int j = 0; j < R; ++j) {
    uint32_t c = 0;
    if (j < nr) {
      const uint64_t bg = gt(j), be = eq(j);
      c = ((uint32_t)__popcll(bg) << 16) | (uint32_t)__popcll(be);
    }
    if (lane == 0) rcnt[j * kW + wave] = c;
  }
  __syncthreads();
  {
    uint32_t total;
    const uint32_t c = tid < R * kW ? rcnt[tid] : 0u;
    const uint32_t ex = block_excl_scan<NT>(c, wsum, total);
    if (tid < R * kW) rcnt[tid] = ex;
    __syncthreads();
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const uint32_t m = remaining;
  int32_t slot[R], src[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    slot[j] = -1;
    src[j] = (int32_t)v[j].y;
    if (j < nr) {
      const uint64_t bg = gt(j), be = eq(j);
      const uint32_t base = rcnt[j * kW + wave];
      const uint32_t gb = (base >> 16) + (uint32_t)__popcll(bg & below);
      const uint32_t eb = (base & 0xFFFFu) + (uint32_t)__popcll(be & below);
      if ((bg >> lane) & 1ull) slot[j] = (int32_t)(gb + (eb < m ? eb : m));
      else if (((be >> lane) & 1ull) && eb < m) slot[j] = (int32_t)(gb + eb);
    }
  }
  emit_slots<R>(row, slot, src, kk);
}

enum SelHow : int32_t { kSelSelf = 1, kSelFull = 2 };

// One workgroup per row.  kSelSelf: the row's level-0 threshold is in ws.thr
// (prefill scan), unless the scan flagged it invalid (thr[3] == 0).
// kSelFull: the workgroup builds the histogram itself.
// Dynamic LDS holds `cap` candidate pairs.  CANDS: candidate rows (the HS
// followers), whose short rows take the early loads below (a separate
// instantiation, so that the other rows keep the smaller register budget).
template <bool CANDS>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkRows a, SelWs ws, int how, int cap) {
  extern __shared__ uint2 cand[];
  __shared__ uint32_t hist[kSelBins];
  constexpr int kRounds = 16;  // collection rounds per chunk
  constexpr int kW = kRowThreads / 64;
  __shared__ uint32_t rcnt[kRounds * kW];
  __shared__ uint32_t wsum[kW];
  __shared__ int32_t sh[4];
  __shared__ uint32_t shb[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  // Candidate rows of at most kRegCand * kRowThreads scores (the HS
  // followers): the scores and the row's candidate positions are loaded
  // first (clamped to its C entries, which the buffers hold), and the row's
  // valid length is counted from those positions instead of searched for.
  const bool early = CANDS && a.C <= kRegCand * kRowThreads;
  uint2 v[kRegCand];
  int32_t mp[kRegCand];
  if (early) {
    const float* sp = a.scores + (int64_t)r * a.C;
    const int32_t* cp = a.cand + (int64_t)(r / a.G) * a.C;
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) {
      const int i = j * kRowThreads + tid;
      const int ic = i < a.C ? i : a.C - 1;
      v[j] = make_uint2(score_key(sp[ic]), (uint32_t)i);
      mp[j] = cp[ic];
    }
  }
  Row row;
  if (early) {
    // Valid candidates come first, then -1 padding: the row's length is the
    // number of non-negative entries, counted from the loaded positions.
    if (tid == 0) sh[0] = 0;
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) c += (uint32_t)__popcll(__ballot(j * kRowThreads + tid < a.C && mp[j] >= 0));
    if ((tid & 63) == 0) atomicAdd(&sh[0], (int32_t)c);
    __syncthreads();
    row.p = a.scores + (int64_t)r * a.C;
    row.n = sh[0];
    row.map = a.cand + (int64_t)(r / a.G) * a.C;
    row.out = a.out + (int64_t)r * a.k;
  } else {
    row = get_row(a, r, sh);
  }
  const int64_t n = row.n;
  const int k = a.k;
  const int64_t kk = n < k ? n : (int64_t)k;
  if (kk == n) {
    keep_all<kRowThreads>(row, n, k);
    return;
  }
  for (int64_t i = kk + tid; i < k; i += kRowThreads) row.out[i] = -1;
  auto gkey = [&](int64_t i) { return score_key(row.p[i]); };
  auto gpos = [&](int64_t i) { return i; };

  // Rows of at most kRegCand * kRowThreads (8192) scores, e.g. the HS
  // followers' candidate rows: every key is loaded once into registers
  // (thread t holds positions t + 512 j, position order), the level-0
  // histogram comes from the registers, and the register selection runs on
  // the whole row (keys below the threshold bin are never kept), instead of
  // a second pass over the row into LDS.
  if (n <= (int64_t)kRegCand * kRowThreads) {
    if (early) {
      // The candidate positions move to the (here unused) dynamic LDS when it
      // holds them (cap pairs >= kRegCand * kRowThreads words), where the final
      // position lookups read them; the barriers of the selection order these
      // writes before those reads.
      if (2 * cap >= kRegCand * kRowThreads) {
        int32_t* lmap = reinterpret_cast<int32_t*>(cand);
#pragma unroll
        for (int j = 0; j < kRegCand; ++j) lmap[j * kRowThreads + tid] = mp[j];
        row.map = lmap;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRegCand; ++j) {
        const int64_t i = (int64_t)j * kRowThreads + tid;
        v[j] = make_uint2(key_clamped(row.p, i, n), (uint32_t)i);
      }
    }
    uint32_t bs, ab;
    const bool own = how == kSelFull || ws.thr[(int64_t)r * 4 + 3] == 0u;
    if (own) {
      for (int i = tid; i < kSelBins; i += kRowThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kRegCand; ++j)
        if ((int64_t)j * kRowThreads + tid < n) atomicAdd(&hist[v[j].x >> kSelShift], 1u);
      __syncthreads();
      constexpr int PER = kSelBins / kRowThreads;
      uint32_t h[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) h[i] = hist[kSelBins - 1 - (tid * PER + i)];
      find_digit<kRowThreads, PER>(h, kSelBins - 1, (uint32_t)kk, wsum, shb);
      bs = shb[0];
      ab = shb[1];
      __syncthreads();  // hist and shb are reused by the selection
    } else {
      bs = ws.thr[(int64_t)r * 4];
      ab = ws.thr[(int64_t)r * 4 + 1];
    }
    select_regs<kRowThreads, kRegCand>(row, v, n, bs << kSelShift, 0xFFE00000u, (uint32_t)kk - ab, kk, hist, wsum,
                                       rcnt, shb);
    return;
  }

  uint32_t bstar, above, eq;
  // kSelSelf rows whose scan histogram overflowed (thr[3] == 0) build it here.
  const bool build = how == kSelFull || ws.thr[(int64_t)r * 4 + 3] == 0u;
  if (build) {
    for (int i = tid; i < kSelBins; i += kRowThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n; b0 += 8LL * kRowThreads) {
      uint32_t kb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t i = b0 + (int64_t)j * kRowThreads + tid;
        kb[j] = key_clamped(row.p, i, n);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (b0 + (int64_t)j * kRowThreads + tid < n) atomicAdd(&hist[kb[j] >> kSelShift], 1u);
    }
    __syncthreads();
    constexpr int PER = kSelBins / kRowThreads;
    uint32_t h[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) h[i] = hist[kSelBins - 1 - (tid * PER + i)];
    find_digit<kRowThreads, PER>(h, kSelBins - 1, (uint32_t)kk, wsum, shb);
    bstar = shb[0];
    above = shb[1];
    eq = shb[2];
  } else {
    const uint32_t* t = ws.thr + (int64_t)r * 4;
    bstar = t[0];
    above = t[1];
    eq = t[2];
  }
  const int64_t nc = (int64_t)above + eq;
  if (nc > cap || above >= (uint32_t)kk) {
    select_keys<kRowThreads>(row, gkey, gpos, n, 0u, 0u, (uint32_t)kk, 0, kk, hist, wsum, shb);
    return;
  }
  // Ordered collection of the keys whose level-0 bin is >= b*: chunks of
  // kRounds * kRowThreads positions; round e of a chunk covers positions
  // base + e*kRowThreads + tid (coalesced), a ballot ranks the kept ones inside
  // each wave, and one scan over the (round, wave) counts places every wave.
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t run = 0;
  // The next chunk's keys are loaded while this one is ranked and stored.
  uint32_t key[kRounds], nkey[kRounds];
  auto load_chunk = [&](uint32_t (&dst)[kRounds], int64_t base) {
#pragma unroll
    for (int e = 0; e < kRounds; ++e) {
      const int64_t i = base + (int64_t)e * kRowThreads + tid;
      dst[e] = key_clamped(row.p, i, n);
    }
  };
  load_chunk(nkey, 0);
#pragma unroll 1
  for (int64_t base = 0; base < n; base += (int64_t)kRounds * kRowThreads) {
    uint64_t ball[kRounds];
#pragma unroll
    for (int e = 0; e < kRounds; ++e) key[e] = nkey[e];
    load_chunk(nkey, base + (int64_t)kRounds * kRowThreads);
#pragma unroll
    for (int e = 0; e < kRounds; ++e) {
      const int64_t i = base + (int64_t)e * kRowThreads + tid;
      ball[e] = __ballot(i < n && (key[e] >> kSelShift) >= bstar);
      if (lane == 0) rcnt[e * kW + wave] = (uint32_t)__popcll(ball[e]);
    }
    __syncthreads();
    uint32_t total;
    static_assert(kRounds * kW <= kRowThreads, "one (round, wave) count per thread");
    const uint32_t cv = tid < kRounds * kW ? rcnt[tid] : 0u;
    const uint32_t ex = block_excl_scan<kRowThreads>(cv, wsum, total);
    if (tid < kRounds * kW) rcnt[tid] = ex;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kRounds; ++e) {
      if ((ball[e] >> lane) & 1ull) {
        const uint32_t pos = run + rcnt[e * kW + wave] + (uint32_t)__popcll(ball[e] & below);
        const int64_t i = base + (int64_t)e * kRowThreads + tid;
        if (pos < (uint32_t)cap) cand[pos] = make_uint2(key[e], (uint32_t)i);
      }
    }
    run += total;
    __syncthreads();  // rcnt is reused
  }
  __syncthreads();
  auto lkey = [&](int64_t i) { return cand[i].x; };
  auto lpos = [&](int64_t i) { return (int64_t)cand[i].y; };
  select_keys<kRowThreads>(row, lkey, lpos, nc, bstar << kSelShift, 0xFFE00000u, (uint32_t)kk - above,
                           1, kk, hist, wsum, shb);
}

constexpr int kListCap = 5632;  // list top-k candidate pairs in LDS at most

// Causal rows given as candidate lists (the prefill scan's output): row r's
// visible positions are 0 .. min(L, qpos0 + r) and its list, list + r * L,
// holds lcnt[r] (key, position) pairs in position order: every visible key
// at or above a floor that never exceeds the row's final threshold bin, so
// the list contains the row's top-k and, for every bin at or above b*, all
// of that bin's keys.  b* comes from the scan (thr) or, when the scan's
// 16-bit histogram overflowed, from a histogram of the list.  One workgroup
// per row; dynamic LDS holds `cap` candidate pairs.
__global__ __launch_bounds__(kRowThreads) void topk_list_kernel(TopkRows a, SelWs ws, const uint2* list_base,
                                                                const uint32_t* lcnt, int cap) {
  extern __shared__ uint2 cand[];
  __shared__ uint32_t hist[kSelBins];
  constexpr int kRounds = 8;  // collection rounds per chunk (16 entries in registers per thread)
  constexpr int kW = kRowThreads / 64;
  __shared__ uint32_t rcnt[kRounds * kW];
  __shared__ uint32_t wsum[kW];
  __shared__ uint32_t shb[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  Row row;
  row.p = nullptr;
  row.map = nullptr;
  row.out = a.out + (int64_t)r * a.k;
  const int64_t vis0 = (int64_t)a.qpos0 + r + 1;
  row.n = vis0 < a.n ? vis0 : a.n;
  const int64_t n = row.n;
  const int k = a.k;
  if (n <= k) {
    keep_all<kRowThreads>(row, n, k);
    return;
  }
  const int64_t kk = k;
  const uint2* list = list_base + (int64_t)r * a.row_stride;
  const int64_t nl = lcnt[r];
  auto lkey = [&](int64_t i) { return list[i].x; };
  auto lpos = [&](int64_t i) { return (int64_t)list[i].y; };

  uint32_t bstar, above, eq;
  if (ws.thr[(int64_t)r * 4 + 3] == 0u) {
    for (int i = tid; i < kSelBins; i += kRowThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < nl; i += kRowThreads) atomicAdd(&hist[list[i].x >> kSelShift], 1u);
    __syncthreads();
    constexpr int PER = kSelBins / kRowThreads;
    uint32_t h[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) h[i] = hist[kSelBins - 1 - (tid * PER + i)];
    find_digit<kRowThreads, PER>(h, kSelBins - 1, (uint32_t)kk, wsum, shb);
    bstar = shb[0];
    above = shb[1];
    eq = shb[2];
  } else {
    const uint32_t* t = ws.thr + (int64_t)r * 4;
    bstar = t[0];
    above = t[1];
    eq = t[2];
  }
  const int64_t nc = (int64_t)above + eq;
  if (nc > cap || above >= (uint32_t)kk) {
    select_keys<kRowThreads>(row, lkey, lpos, nl, 0u, 0u, (uint32_t)kk, 0, kk, hist, wsum, shb);
    return;
  }
  // Ordered collection of the list entries whose level-0 bin is >= b*, as in
  // topk_row_kernel: chunks of kRounds * kRowThreads entries, a ballot per
  // round and one scan over the (round, wave) counts.
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t run = 0;
  uint2 e[kRounds], ne[kRounds];
  auto load_chunk = [&](uint2 (&dst)[kRounds], int64_t base) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t i = base + (int64_t)j * kRowThreads + tid;
      dst[j] = list[i < nl ? i : nl - 1];  // clamped, branch-free (nl >= k >= 1 here)
    }
  };
  load_chunk(ne, 0);
#pragma unroll 1
  for (int64_t base = 0; base < nl; base += (int64_t)kRounds * kRowThreads) {
    uint64_t ball[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) e[j] = ne[j];
    load_chunk(ne, base + (int64_t)kRounds * kRowThreads);
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t i = base + (int64_t)j * kRowThreads + tid;
      ball[j] = __ballot(i < nl && (e[j].x >> kSelShift) >= bstar);
      if (lane == 0) rcnt[j * kW + wave] = (uint32_t)__popcll(ball[j]);
    }
    __syncthreads();
    uint32_t total;
    const uint32_t cv = tid < kRounds * kW ? rcnt[tid] : 0u;
    const uint32_t ex = block_excl_scan<kRowThreads>(cv, wsum, total);
    if (tid < kRounds * kW) rcnt[tid] = ex;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if ((ball[j] >> lane) & 1ull) {
        const uint32_t pos = run + rcnt[j * kW + wave] + (uint32_t)__popcll(ball[j] & below);
        if (pos < (uint32_t)cap) cand[pos] = e[j];
      }
    }
    run += total;
    __syncthreads();  // rcnt is reused
  }
  __syncthreads();
  auto ckey = [&](int64_t i) { return cand[i].x; };
  auto cpos = [&](int64_t i) { return (int64_t)cand[i].y; };
  select_keys<kRowThreads>(row, ckey, cpos, nc, bstar << kSelShift, 0xFFE00000u, (uint32_t)kk - above, 1, kk, hist,
                           wsum, shb);
}

// One workgroup per (segment, row); see the file comment.  Dynamic LDS holds
// the last workgroup's candidates (ws.cap pairs).
// SEGPER: positions per thread in a segment (segment = SEGPER * kSegThreads).
template <int SEGPER>
__global__ __launch_bounds__(kSegThreads) void topk_segmented_kernel(TopkRows a, SelWs ws) {
  constexpr int kSegPer = SEGPER;
  constexpr int kSegLen = SEGPER * kSegThreads;
  extern __shared__ uint2 lcand[];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wsum[kSegThreads / 64];
  __shared__ uint32_t segoff[kSegThreads];
  __shared__ int32_t sh[4];
  __shared__ uint32_t shb[4];
  __shared__ int32_t sh_last;
  const int tid = threadIdx.x;
  const int r = blockIdx.y, s = blockIdx.x;
  const Row row = get_row(a, r, sh);
  const int64_t n = row.n;
  const int k = a.k;
  if (n <= k) {
    if (s == 0) keep_all<kSegThreads>(row, n, k);
    return;
  }
  int64_t nseg_row = (n + kSegLen - 1) / kSegLen;
  nseg_row = nseg_row < ws.nseg ? nseg_row : ws.nseg;
  if (s >= nseg_row) return;

  // The segment's scores are loaded first: their latency overlaps the
  // reduction of the partial histograms below.  Round e covers positions
  // s0 + NT*e + tid (coalesced).
  const int64_t s0 = (int64_t)s * kSegLen;
  const int64_t s1 = (s0 + kSegLen) < n ? (s0 + kSegLen) : n;
  const int slen = (int)(s1 - s0);  // segment-local indices are 32-bit
  const float* sp = row.p + s0;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kW = kSegThreads / 64;
  uint32_t key[kSegPer];
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const int ii = e * kSegThreads + tid;  // clamped, branch-free (ignored past the end)
    key[e] = score_key(sp[ii < slen ? ii : slen - 1]);
  }

  // 1. Threshold bin b* from the row's partial histograms (16-bit, one per
  //    scan workgroup), in two small reads: the coarse partials (64 bins of
  //    32) give the coarse bin holding the k-th key, then only its 32 fine
  //    bins are read from each partial.  hist[] is the reduction scratch.
  int64_t nw = (n + ws.chunk - 1) / ws.chunk;
  nw = nw < ws.nwg ? nw : ws.nwg;
  const int64_t prow = (int64_t)r * ws.nwg;
  {
    constexpr int kCG = kSegThreads / kSelCoarse;  // partial groups in the coarse pass
    const int c = tid % kSelCoarse, grp = tid / kSelCoarse;
    uint32_t cs = 0;
#pragma unroll 1
    for (int64_t w0 = grp; w0 < nw; w0 += 4 * kCG) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t wj = w0 + (int64_t)j * kCG;
        v[j] = ws.cpart[(prow + (wj < nw ? wj : nw - 1)) * kSelCoarse + c];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) cs += (w0 + (int64_t)j * kCG < nw) ? v[j] : 0u;
    }
    hist[grp * kSelCoarse + c] = cs;
    __syncthreads();
    if (wave == 0) {
      // lane i: coarse bin 63 - i (descending order)
      const int cb = kSelCoarse - 1 - lane;
      uint32_t h = 0;
#pragma unroll
      for (int gI = 0; gI < kCG; ++gI) h += hist[gI * kSelCoarse + cb];
      const uint32_t incl = wave_incl_scan(h);
      if (incl - h < (uint32_t)k && incl >= (uint32_t)k) {
        shb[0] = (uint32_t)cb;
        shb[1] = incl - h;
      }
    }
    __syncthreads();
  }
  const uint32_t cstar = shb[0], cabove = shb[1];
  __syncthreads();
  {
    constexpr int kFG = kSegThreads / kSelFine;  // partial groups in the fine pass
    const int i = tid % kSelFine, grp = tid / kSelFine;
    const int bin = (int)cstar * kSelFine + i;
    uint32_t fs = 0;
#pragma unroll 1
    for (int64_t w0 = grp; w0 < nw; w0 += 4 * kFG) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t wj = w0 + (int64_t)j * kFG;
        v[j] = ws.part[(prow + (wj < nw ? wj : nw - 1)) * kSelBins + bin];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) fs += (w0 + (int64_t)j * kFG < nw) ? v[j] : 0u;
    }
    hist[grp * kSelFine + i] = fs;
    __syncthreads();
    if (wave == 0) {
      // lane i < 32: fine bin 32 c* + 31 - i (descending), after cabove keys
      const int fb = kSelFine - 1 - lane;
      uint32_t h = 0;
      if (lane < kSelFine) {
#pragma unroll
        for (int gI = 0; gI < kFG; ++gI) h += hist[gI * kSelFine + fb];
      }
      const uint32_t incl = cabove + wave_incl_scan(h);
      if (lane < kSelFine && incl - h < (uint32_t)k && incl >= (uint32_t)k) {
        shb[0] = cstar * kSelFine + (uint32_t)fb;
        shb[1] = incl - h;
        shb[2] = h;
      }
    }
    __syncthreads();
  }
  const uint32_t bstar = shb[0], above = shb[1], eq = shb[2];

  // 2. This segment's candidates, in position order: within a wave the kept
  //    positions are ranked with a ballot, and one scan over the (round, wave)
  //    counts gives every wave its output offset per round.
  // The ballots are taken again in the write pass rather than kept (64 bits
  // per round would hold 2 kSegPer more registers across the scan).
  auto keep = [&](int e) { return __ballot(e * kSegThreads + tid < slen && (key[e] >> kSelShift) >= bstar); };
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const uint64_t b = keep(e);
    if (lane == 0) segoff[e * kW + wave] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  uint32_t total;
  {
    static_assert(kSegPer * kW <= kSegThreads, "one (round, wave) count per thread");
    const uint32_t v = tid < kSegPer * kW ? segoff[tid] : 0u;
    const uint32_t ex = block_excl_scan<kSegThreads>(v, wsum, total);
    if (tid < kSegPer * kW) segoff[tid] = ex;
    __syncthreads();
  }
  // Candidates and counts are published with agent-scope atomic stores,
  // which write through the (per-XCD, non-coherent) L2, and read back the same
  // way by the finishing workgroup.  One release per workgroup (step 3) orders
  // them; a __threadfence() in every thread would write back the L2 once per
  // wave instead.
  uint64_t* dst = reinterpret_cast<uint64_t*>(ws.cand + ((int64_t)r * ws.nseg + s) * kSegLen);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const uint64_t b = keep(e);
    if ((b >> lane) & 1ull) {
      const uint32_t pos = segoff[e * kW + wave] + (uint32_t)__popcll(b & below);
      const uint32_t i = (uint32_t)s0 + (uint32_t)(e * kSegThreads + tid);
      const uint64_t pr = (uint64_t)key[e] | ((uint64_t)i << 32);
      __hip_atomic_store(dst + pos, pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (tid == 0)
    __hip_atomic_store(ws.cnt + (int64_t)r * ws.nseg + s, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 3. The last segment of the row to finish does the final selection.
  //    Ordering of the hand-off (AMDGPU memory model, agent scope):
  //    - every wave waits for its own candidate and count stores to complete
  //      (s_waitcnt 0) before the barrier, so the workgroup's stores are done
  //      when the counter moves, whatever the barrier's fences imply;
  //    - the barrier makes them happen-before tid 0's agent-scope release
  //      fence (L2 write-back), which completes before the counter update;
  //    - the workgroup that reads the final count does an agent-scope acquire
  //      (L1/L2 invalidate) before the barrier that lets its other waves read
  //      the candidates, so it observes every releasing workgroup's stores.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // also: segoff is reused below
  if (tid == 0) {
    // Release fence, then an explicit wait: the write-back must be complete
    // before the counter moves (the compiler's own wait after the write-back
    // is dropped when no store is pending).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
    const bool last = __hip_atomic_fetch_add(ws.done + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
                      (uint32_t)nseg_row;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sh_last = last;
  }
  __syncthreads();
  if (!sh_last) return;
  if (tid == 0) __hip_atomic_store(ws.done + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const int64_t kk = k;
  const int64_t nc = (int64_t)above + eq;
  auto gkey = [&](int64_t i) { return score_key(row.p[i]); };
  auto gpos = [&](int64_t i) { return i; };
  if (above >= (uint32_t)kk || nseg_row > kSegThreads) {
    select_keys<kSegThreads>(row, gkey, gpos, n, 0u, 0u, (uint32_t)kk, 0, kk, hist, wsum, shb);
    return;
  }
  // Segment offsets of the candidate lists.
  const uint32_t cs = tid < nseg_row ? __hip_atomic_load(ws.cnt + (int64_t)r * ws.nseg + tid, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                     : 0u;
  uint32_t ctot;
  const uint32_t co = block_excl_scan<kSegThreads>(cs, wsum, ctot);
  if (tid < nseg_row) segoff[tid] = co;
  __syncthreads();
  const int64_t ncl = (int64_t)ctot < nc ? (int64_t)ctot : nc;
  auto seg_of = [&](int64_t i) {
    int lo = 0, hi = (int)nseg_row - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (segoff[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto gcand = [&](int64_t i) {
    const int sg = seg_of(i);
    uint64_t* p = reinterpret_cast<uint64_t*>(ws.cand + ((int64_t)r * ws.nseg + sg) * kSegLen + (i - segoff[sg]));
    const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
  };
  const uint32_t pfx = bstar << kSelShift, pmask = 0xFFE00000u, rem = (uint32_t)kk - above;
  if (ncl <= (int64_t)kRegCand * kSegThreads) {
    // Thread t loads candidates t + 512 j; its positions only grow, so its
    // segment is tracked with a cursor that moves forward.  Indices past the
    // end load the last candidate (branch-free loads), which is ignored.
    int sg = seg_of(tid < ncl ? tid : ncl - 1);
    uint32_t cur = segoff[sg];
    uint32_t nxt = sg + 1 < nseg_row ? segoff[sg + 1] : 0xFFFFFFFFu;
    uint2 v[kRegCand];
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) {
      const int64_t i = (int64_t)j * kSegThreads + tid;
      const uint32_t ic = (uint32_t)(i < ncl ? i : ncl - 1);
      while (ic >= nxt) {
        ++sg;
        cur = nxt;
        nxt = sg + 1 < nseg_row ? segoff[sg + 1] : 0xFFFFFFFFu;
      }
      uint64_t* p = reinterpret_cast<uint64_t*>(ws.cand + ((int64_t)r * ws.nseg + sg) * kSegLen + (ic - cur));
      const uint64_t x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v[j] = make_uint2((uint32_t)x, (uint32_t)(x >> 32));
    }
    __syncthreads();  // segoff is reused as the compaction's count table
    select_regs<kSegThreads, kRegCand>(row, v, ncl, pfx, pmask, rem, kk, hist, wsum, segoff, shb);
  } else if (ncl <= ws.cap) {
    // Batches of kBatch independent loads per thread, so their latencies
    // overlap.  A thread's positions only grow, so its segment is tracked with
    // a cursor that moves forward (next segment start cached in a register).
    constexpr int kBatch = 16;
    int sg = seg_of(tid < ncl ? tid : ncl - 1);
    uint32_t cur = segoff[sg];
    uint32_t nxt = sg + 1 < nseg_row ? segoff[sg + 1] : 0xFFFFFFFFu;
#pragma unroll 1
    for (int64_t b0 = 0; b0 < ncl; b0 += (int64_t)kBatch * kSegThreads) {
      uint2 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        // Clamped to the last candidate (branch-free load; repeats are not stored).
        const int64_t i = b0 + (int64_t)j * kSegThreads + tid;
        const uint32_t ic = (uint32_t)(i < ncl ? i : ncl - 1);
        while (ic >= nxt) {
          ++sg;
          cur = nxt;
          nxt = sg + 1 < nseg_row ? segoff[sg + 1] : 0xFFFFFFFFu;
        }
        uint64_t* p = reinterpret_cast<uint64_t*>(ws.cand + ((int64_t)r * ws.nseg + sg) * kSegLen + (ic - cur));
        const uint64_t x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[j] = make_uint2((uint32_t)x, (uint32_t)(x >> 32));
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = b0 + (int64_t)j * kSegThreads + tid;
        if (i < ncl) lcand[i] = v[j];
      }
    }
    __syncthreads();
    auto lkey = [&](int64_t i) { return lcand[i].x; };
    auto lpos = [&](int64_t i) { return (int64_t)lcand[i].y; };
    select_keys<kSegThreads>(row, lkey, lpos, ncl, pfx, pmask, rem, 1, kk, hist, wsum, shb);
  } else {
    auto ckey = [&](int64_t i) { return gcand(i).x; };
    auto cpos = [&](int64_t i) { return (int64_t)gcand(i).y; };
    select_keys<kSegThreads>(row, ckey, cpos, ncl, pfx, pmask, rem, 1, kk, hist, wsum, shb);
  }
}

// Bucket mode (decode): one workgroup per row, reading what the scan left
// (SelWs::bucket).  Summing the scan workgroups' descending prefix counts
// gives Q[b], the row's keys in bins >= b, so the threshold bin b* (Q[b*] >= k
// > Q[b*+1]) needs no scan; list w holds its keys in bins > b* first
// (part_w[b*+1] of them), then those in b* (up to part_w[b*]).  The lists'
// first entries are loaded together with the partials (one round trip; the
// rest, where a list holds more, afterwards).  Keys above b* are all kept:
// their positions are marked in a bitmap and kept as 4-byte positions.  Only
// the keys in b* go through two more radix levels, which give the k-th key T
// and the number m of keys equal to T that fit; those are marked in the
// bitmaps (> T, == T) too.  With per-word prefix counts of the bitmaps every
// kept position finds its place in position order,
//   slot = #greater-before + min(#equal-before, m),
// in an LDS copy of the output row (k <= kBucketStageK; beyond, straight to
// the output).  Dynamic LDS: ecap (key, position) pairs of bin b*, k
// positions above it, the two bitmaps and the word prefixes (nwords each),
// then the staged row.  A bin b* beyond ecap is read from global memory.
constexpr int kBucketThreads = 512;

template <int NT, typename KeyAt, typename PosAt>
__device__ void bucket_finish(const Row& row, KeyAt key_at, PosAt pos_at, uint32_t neq, const uint32_t* gpos,
                              uint32_t ngt, uint32_t bstar, int64_t kk, int64_t n, uint32_t* gbits, uint32_t* ebits,
                              uint32_t* wpre, uint32_t* stage, uint32_t* hist, uint32_t* wsum, uint32_t* shb) {
  const int tid = threadIdx.x;
  uint32_t prefix = bstar << kSelShift, pmask = 0xFFE00000u, rem = (uint32_t)kk - ngt, cnt = neq;
#pragma unroll 1
  for (int level = 1; level < 3 && cnt != rem; ++level) {
    const int shift = level == 1 ? 10 : 0;
    const int nb = level == 1 ? kSelBins : kSelBins / 2;
    radix_level<NT>(key_at, (int64_t)neq, prefix, pmask, shift, nb, rem, hist, wsum, shb);
    prefix |= shb[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    rem -= shb[1];
    cnt = shb[2];
    __syncthreads();
  }
  LI_STAMP(5);
  // Keys of b* above the resolved prefix are kept; of those equal to it, the
  // first rem by position.
#pragma unroll 1
  for (uint32_t e = tid; e < neq; e += NT) {
    const uint32_t key = key_at(e) & pmask;
    const uint32_t p = (uint32_t)pos_at(e);
    if (key > prefix) atomicOr(&gbits[p >> 5], 1u << (p & 31));
    else if (key == prefix) atomicOr(&ebits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  LI_STAMP(6);
  // Per bitmap word, the marked positions before it: #greater << 18 | #equal
  // (#greater < k <= 2^14, #equal <= n <= 2^17).  Wave v takes words
  // [v*WPW, (v+1)*WPW) in rounds of 64 consecutive words (one per lane, no
  // bank conflicts), scans each round within the wave and keeps a running
  // total; the waves' totals then give each wave its offset.
  // All of a wave's bitmap reads are issued before its first scan, and the
  // wave's offset is added in registers, so each word's prefix is written once.
  constexpr int NWV = NT / 64;
  constexpr int WR = (kBucketMaxLen / 32 + NT - 1) / NT;  // rounds of 64 words per wave at most
  const int nwr = (int)((n + 31) / 32);
  const int WPW = ((nwr + NWV - 1) / NWV + 63) / 64 * 64;  // <= 64 * WR
  const int wv = tid >> 6, ln = tid & 63;
  uint32_t cw[WR], iw[WR];
#pragma unroll
  for (int i = 0; i < WR; ++i) {
    const int w = wv * WPW + 64 * i + ln;
    const bool in = 64 * i < WPW && w < nwr;
    const int wc = in ? w : 0;
    const uint32_t gb = gbits[wc], eb = ebits[wc];
    cw[i] = in ? ((uint32_t)__builtin_popcount(gb) << 18) + (uint32_t)__builtin_popcount(eb) : 0u;
  }
  uint32_t run = 0;
#pragma unroll
  for (int i = 0; i < WR; ++i) {
    const uint32_t inc = wave_incl_scan(cw[i]);
    iw[i] = run + inc - cw[i];
    run += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  }
  if (ln == 0) wsum[wv] = run;
  __syncthreads();
  uint32_t woff = 0;
  for (int v = 0; v < NWV; ++v) woff += v < wv ? wsum[v] : 0u;
#pragma unroll
  for (int i = 0; i < WR; ++i) {
    const int w = wv * WPW + 64 * i + ln;
    if (64 * i < WPW && w < nwr) wpre[w] = woff + iw[i];
  }
  __syncthreads();
  LI_STAMP(7);
  // Every kept position's slot: #greater-before + min(#equal-before, m), or for
  // an equal key #greater-before + #equal-before when that is below m.
  const uint32_t m = rem;
  auto place = [&](uint32_t p, bool greater) {
    const uint32_t w = p >> 5, below = (1u << (p & 31)) - 1u;
    const uint32_t pre = wpre[w];
    const uint32_t gb = (pre >> 18) + (uint32_t)__builtin_popcount(gbits[w] & below);
    const uint32_t eb = (pre & 0x3FFFFu) + (uint32_t)__builtin_popcount(ebits[w] & below);
    const uint32_t slot = greater ? gb + (eb < m ? eb : m) : (eb < m ? gb + eb : 0xFFFFFFFFu);
    if (slot < (uint32_t)kk) {
      if (stage) stage[slot] = p;
      else row.out[slot] = (int32_t)p;
    }
  };
#pragma unroll 1
  for (uint32_t e = tid; e < ngt; e += NT) place(gpos[e], true);
#pragma unroll 1
  for (uint32_t e = tid; e < neq; e += NT) {
    const uint32_t key = key_at(e) & pmask;
    if (key >= prefix) place((uint32_t)pos_at(e), key > prefix);
  }
  if (stage) {
    __syncthreads();
    LI_STAMP(8);
    for (int i = tid; i < kk; i += NT) row.out[i] = (int32_t)stage[i];
  } else {
    LI_STAMP(8);  // (slots written straight to the output: thread 0's own progress)
  }
  LI_STAMP(9);
}

// NWMAX: scan workgroups per request at most; RS: list entries per thread in
// the up-front loads.
template <int NWMAX, int RS>
__global__ __launch_bounds__(kBucketThreads) void topk_bucket_kernel(TopkRows a, SelWs ws, int ecap, int nwords,
                                                                     int staged) {
  constexpr int NT = kBucketThreads;
  static_assert(4 * NT == kSelBins, "four level-0 bins per thread");
  constexpr int TPC = NT / NWMAX;              // threads per list in the up-front loads
  constexpr int SPW = TPC * RS;                // entries per list loaded up front (128 .. 384)
  extern __shared__ uint2 bdyn[];
  const int k = a.k;
  uint2* eqc = bdyn;
  uint32_t* gpos = reinterpret_cast<uint32_t*>(bdyn + ecap);
  uint32_t* gbits = gpos + k;
  uint32_t* ebits = gbits + nwords;
  uint32_t* wpre = ebits + nwords;
  uint32_t* stage = staged ? wpre + nwords : nullptr;
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t qfirst[NT], qlast[NT];
  __shared__ uint32_t cge[NWMAX], cgt[NWMAX];  // per list: keys in bins >= b*, in bins > b*
  __shared__ uint32_t gstart[NWMAX + 1], estart[NWMAX + 1];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t shb[4];
  __shared__ int32_t sh[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int64_t prow = (int64_t)r * ws.nwg;
  LI_STAMP(0);
  // 1. One round of loads, issued before the row's length is known (so they
  //    do not wait for kv_off): the 8 bytes of bins 4t .. 4t+3 of every
  //    partial, and entries sl + TPC*j of list sw.  Indices are clamped to the
  //    workspace, not branched on; partials and list slots that the scan did
  //    not write this call (past the row's end) are loaded and ignored.
  const int sw = tid / TPC, sl = tid % TPC;
  const uint2* slist = ws.blist + (prow + (sw < ws.nwg ? sw : ws.nwg - 1)) * ws.chunk;
  // Two entries per 16-byte load: entries 2 (sl + TPC j) and 2 (sl + TPC j) + 1.
  static_assert(RS % 2 == 0, "entry pairs");
  i32x4 sv[RS / 2];
#pragma unroll
  for (int j = 0; j < RS / 2; ++j) sv[j] = ld16(slist + 2 * (sl + TPC * j));
  uint2 pw[NWMAX];
#pragma unroll
  for (int w = 0; w < NWMAX; ++w) {
    const int wc = w < ws.nwg ? w : ws.nwg - 1;
    pw[w] = *reinterpret_cast<const uint2*>(ws.part + (prow + wc) * kSelBins + 4 * tid);
  }
  const Row row = get_row(a, r, sh);
  const int64_t n = row.n;
  if (n <= k) {
    keep_all<NT>(row, n, k);
    return;
  }
  const int nw = (int)((n + ws.chunk - 1) / ws.chunk);  // <= ws.nwg <= NWMAX (host-checked)
  const int nwr = (int)((n + 31) / 32);
  for (int i = tid; i < nwr; i += NT) {
    gbits[i] = 0u;
    ebits[i] = 0u;
  }
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  auto half = [&](const uint2& v, int i) {
    const uint32_t word = i < 2 ? v.x : v.y;
    return (i & 1) ? (word >> 16) : (word & 0xFFFFu);
  };
#pragma unroll
  for (int w = 0; w < NWMAX; ++w) {
    if (w < nw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] += half(pw[w], i);
    }
  }
  qfirst[tid] = q[0];
  qlast[tid] = q[3];
  __syncthreads();
  LI_STAMP(1);
  {
    // Q is non-increasing with Q[0] = n > k and Q[2048] = 0: one bin crosses.
    // Its thread records part_w[b*] and, but for the last bin of its four,
    // part_w[b*+1]; in that case the next thread records the latter.
    const uint32_t kk = (uint32_t)k;
    const uint32_t qn = tid + 1 < NT ? qfirst[tid + 1] : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qa = q[i], qb = i < 3 ? q[i + 1] : qn;
      if (qa >= kk && qb < kk) {
        shb[0] = (uint32_t)(4 * tid + i);
        shb[1] = qb;
        shb[2] = qa - qb;
#pragma unroll
        for (int w = 0; w < NWMAX; ++w) {
          if (w < nw) {
            cge[w] = half(pw[w], i);
            if (i < 3) cgt[w] = half(pw[w], i + 1);
            else if (tid == NT - 1) cgt[w] = 0u;
          }
        }
      }
    }
    if (tid > 0 && q[0] < kk && qlast[tid - 1] >= kk) {
#pragma unroll
      for (int w = 0; w < NWMAX; ++w)
        if (w < nw) cgt[w] = half(pw[w], 0);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const uint32_t g = tid < nw ? cgt[tid] : 0u, e = tid < nw ? cge[tid] - cgt[tid] : 0u;
    const uint32_t gi = wave_incl_scan(g), ei = wave_incl_scan(e);
    if (tid < nw) {
      gstart[tid + 1] = gi;
      estart[tid + 1] = ei;
    }
    if (tid == 0) {
      gstart[0] = 0u;
      estart[0] = 0u;
    }
  }
  __syncthreads();
  LI_STAMP(2);
  const uint32_t bstar = shb[0], ngt = shb[1], neq = shb[2];
  __syncthreads();  // shb is reused by the radix levels
  const bool eq_lds = neq <= (uint32_t)ecap;

  // 2. Entry e of list w: below cgt[w] a key above b* (its position is kept
  //    and marked), below cge[w] a key of b* (into LDS when they fit).
  if (sw < nw) {
    const uint32_t cw = cge[sw], gw = cgt[sw], gb = gstart[sw], eb = estart[sw];
    auto put = [&](uint32_t e, const uint2& v) {
      if (e < gw) {
        gpos[gb + e] = v.y;
        atomicOr(&gbits[v.y >> 5], 1u << (v.y & 31));
      } else if (e < cw && eq_lds) {
        eqc[eb + (e - gw)] = v;
      }
    };
#pragma unroll
    for (int j = 0; j < RS / 2; ++j) {
      put((uint32_t)(2 * (sl + TPC * j)), make_uint2((uint32_t)sv[j].x, (uint32_t)sv[j].y));
      put((uint32_t)(2 * (sl + TPC * j) + 1), make_uint2((uint32_t)sv[j].z, (uint32_t)sv[j].w));
    }
    // the rest of a long list, eight loads per thread at a time
#pragma unroll 1
    for (uint32_t e0 = (uint32_t)(SPW + sl); e0 < cw; e0 += 8 * TPC) {
      uint2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = e0 + TPC * j;
        v[j] = slist[e < cw ? e : cw - 1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = e0 + TPC * j;
        if (e < cw) put(e, v[j]);
      }
    }
  }
  __syncthreads();
  LI_STAMP(3);
  if (eq_lds) {
    auto lkey = [&](int64_t e) { return eqc[e].x; };
    auto lpos = [&](int64_t e) { return (int64_t)eqc[e].y; };
    bucket_finish<NT>(row, lkey, lpos, neq, gpos, ngt, bstar, k, n, gbits, ebits, wpre, stage, hist, wsum, shb);
  } else {
    // Entry e of bin b*: list w with estart[w] <= e < estart[w+1], at cgt[w] + (e - estart[w]).
    auto gcand = [&](int64_t e) {
      int lo = 0, hi = nw - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (estart[mid] <= (uint32_t)e) lo = mid; else hi = mid - 1;
      }
      return ws.blist[(prow + lo) * ws.chunk + cgt[lo] + ((uint32_t)e - estart[lo])];
    };
    auto gkey = [&](int64_t e) { return gcand(e).x; };
    auto gpos_at = [&](int64_t e) { return (int64_t)gcand(e).y; };
    bucket_finish<NT>(row, gkey, gpos_at, neq, gpos, ngt, bstar, k, n, gbits, ebits, wpre, stage, hist, wsum, shb);
  }
}

}  // namespace

int64_t seg_len_for(int64_t rows, int64_t max_len) {
  // One round of segment workgroups on the GPU (2 per CU at the default LDS
  // size); beyond that, twice as many scores per workgroup.
  const int64_t nseg = (max_len + kSeg - 1) / kSeg;
  return rows * nseg > 512 ? 2 * kSeg : kSeg;
}

int32_t seg_cap_for(int32_t k) {
  // The candidates are the keys above the threshold bin (fewer than k) plus the
  // whole threshold bin, a quarter of an octave of score values that can hold
  // thousands of keys near the cut (rows of 128K LatentIndex scores put up to
  // ~4.3K there at k = 2048).  8192 pairs still leave room for two workgroups
  // per CU; rows beyond the cap take the slower global-memory path.
  const int64_t a = 2 * (int64_t)k + 2048, b = 4 * (int64_t)k;
  const int64_t cap = a > b ? a : b;
  return (int32_t)(cap < kMaxCap ? cap : kMaxCap);
}

// Dynamic LDS beyond the default 64 KB needs a one-time opt-in per kernel.
template <typename K>
hipError_t allow_lds(K kernel, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     kMaxCap * (int)sizeof(uint2));
  if (e == hipSuccess) done = true;
  return e;
}

hipError_t launch_topk_segmented(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const int nseg = ws.nseg > 0 ? ws.nseg : 1;
  const dim3 grid((unsigned)nseg, (unsigned)a.rows);
  // Candidate sets up to kRegCand * kSegThreads stay in registers; the LDS
  // buffer is only allocated for larger caps (k above 2048).
  SelWs w = ws;
  if (w.cap <= kRegCand * kSegThreads) w.cap = 0;
  const size_t lds = (size_t)w.cap * sizeof(uint2);
  if (w.seg == 2 * kSeg) {
    static bool lds_set = false;
    if (hipError_t e = allow_lds(topk_segmented_kernel<2 * kSeg / kSegThreads>, lds_set)) return e;
    return launch_kernel(topk_segmented_kernel<2 * kSeg / kSegThreads>, grid, dim3(kSegThreads), (uint32_t)lds,
                         stream, a, w);
  }
  static bool lds_set = false;
  if (hipError_t e = allow_lds(topk_segmented_kernel<kSeg / kSegThreads>, lds_set)) return e;
  return launch_kernel(topk_segmented_kernel<kSeg / kSegThreads>, grid, dim3(kSegThreads), (uint32_t)lds, stream,
                       a, w);
}

static hipError_t launch_row(const TopkRows& a, const SelWs& ws, int how, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const int cap = seg_cap_for(a.k);
  if (a.mode == kRowsCands) {
    static bool lds_set = false;
    if (hipError_t e = allow_lds(topk_row_kernel<true>, lds_set)) return e;
    return launch_kernel(topk_row_kernel<true>, dim3((unsigned)a.rows), dim3(kRowThreads),
                         (uint32_t)(cap * sizeof(uint2)), stream, a, ws, how, cap);
  }
  static bool lds_set = false;
  if (hipError_t e = allow_lds(topk_row_kernel<false>, lds_set)) return e;
  return launch_kernel(topk_row_kernel<false>, dim3((unsigned)a.rows), dim3(kRowThreads),
                       (uint32_t)(cap * sizeof(uint2)), stream, a, ws, how, cap);
}

hipError_t launch_topk_self(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  return launch_row(a, ws, kSelSelf, stream);
}

hipError_t launch_topk_list(const TopkRows& a, const SelWs& ws, const uint2* list, const uint32_t* lcnt,
                            hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  static bool lds_set = false;
  if (hipError_t e = allow_lds(topk_list_kernel, lds_set)) return e;
  // Three workgroups per CU (68 VGPRs, 8.3 KB of static LDS): the candidate
  // room is capped at 5632 pairs (44 KB); rows with more take the global path.
  const int cap = seg_cap_for(a.k) < kListCap ? seg_cap_for(a.k) : kListCap;
  return launch_kernel(topk_list_kernel, dim3((unsigned)a.rows), dim3(kRowThreads), (uint32_t)(cap * sizeof(uint2)),
                       stream, a, ws, list, lcnt, cap);
}

// LDS of the bucket top-k besides the (key, position) pairs of bin b*: k
// positions above b*, two bitmaps and the word prefixes, and the staged
// output row when k <= kBucketStageK.
static int64_t bucket_fixed_lds(int32_t k, int64_t max_len) {
  return 4 * (int64_t)k + 3 * ((max_len + 31) / 32) * 4 + (k <= kBucketStageK ? 4 * (int64_t)k : 0);
}

int32_t bucket_cap_for(int32_t k, int64_t max_len) {
  const int64_t room = (kBucketLds - bucket_fixed_lds(k, max_len)) / 8;
  return (int32_t)(room > 0 ? room : 0);
}

bool bucket_ok(int64_t nwg, int64_t chunk, int32_t k, int64_t max_len) {
  // The scan's lists must fit its LDS staging (every key when the workgroup
  // holds at most 4096, else the floor must leave out at least half), and the
  // selection needs useful room for the keys of the threshold bin.
  return nwg >= 1 && nwg <= kBucketMaxNwg && max_len <= kBucketMaxLen &&
         (2 * (int64_t)k <= chunk || chunk <= 4096) && bucket_cap_for(k, max_len) >= 1024;
}

hipError_t launch_topk_bucket(const TopkRows& a, const SelWs& ws, int64_t max_len, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  const int ecap = bucket_cap_for(a.k, max_len);
  const int nwords = (int)((max_len + 31) / 32);
  const int staged = a.k <= kBucketStageK ? 1 : 0;
  const uint32_t lds = (uint32_t)ecap * 8u + (uint32_t)bucket_fixed_lds(a.k, max_len);
  // Up-front list loads: a request's lists hold k keys above b* and the keys
  // of b* itself (about 3K in all at k = 2048 over 128K positions), so 16
  // lists take 256 entries each and 32 lists 128 each at k <= 2048; a larger k
  // loads 384 per list.  The rest of a longer list follows in a second round.
  auto go = [&](auto kernel, bool& lds_set) -> hipError_t {
    if (!lds_set) {
      if (hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kBucketLds))
        return e;
      lds_set = true;
    }
    return launch_kernel(kernel, dim3((unsigned)a.rows), dim3(kBucketThreads), lds, stream, a, ws, ecap, nwords,
                         staged);
  };
  static bool set16 = false, set32s = false, set32 = false;
  if (ws.nwg <= 16) return go(topk_bucket_kernel<16, 8>, set16);
  if (a.k <= 2048) return go(topk_bucket_kernel<kBucketMaxNwg, 8>, set32s);
  return go(topk_bucket_kernel<kBucketMaxNwg, 24>, set32);
}

hipError_t launch_topk(const TopkRows& a, hipStream_t stream) {
  SelWs none = {};
  return launch_row(a, none, kSelFull, stream);
}

#ifdef LI_STAMPS
// Copies the stamps of the last bucket top-k call (rows < 64, 10 phases each,
// 100 MHz ticks) to host memory; 0 on success.
extern "C" int li_read_stamps(unsigned long long* host, int n) {
  if (!host || n < 0 || n > kStampRows * kStampPhases) return -1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(li_stamp_buf), (size_t)n * 8) == hipSuccess ? 0 : -1;
}
#endif

}  // namespace li
