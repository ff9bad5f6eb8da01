// Per-row top-k selection on gfx950 (the step that turns indexer scores into
// the index tensor: "IndexCache: Cross-Layer Index Reuse for Sparse
// Attention", Deep Dive, the F layer takes top-k of its scores).
//
// Scores map to order-preserving uint32 keys (-0 folded onto +0).  The
// selection is a radix select whose first level (the top 11 key bits) is a
// histogram that the scan kernels build while they write the scores, so the
// threshold bin b* -- the level-0 bin holding the k-th largest key -- is known
// before the selection starts ("pre" mode: the scan workgroups store partial
// histograms that hist_reduce sums per row).  Then:
//   collect (many workgroups per row, "pre" mode): each 8192-score segment of a
//     row keeps, in position order, the (key, position) pairs whose bin is
//     >= b*; at most (k-1) + |b*| of them exist in the whole row.
//   final (one workgroup per row): loads those candidates into LDS in position
//     order (or collects them itself in "self" mode, or first builds the
//     level-0 histogram itself in "full" mode), resolves the remaining 21 key
//     bits among the keys of bin b* with two more LDS histogram levels, and
//     writes the kept positions with an ordered compaction:
//       slot = #greater-before + min(#equal-before, m),
//     where m is how many keys equal to the k-th key still fit -- so the output
//     is in ascending position order and the lower position wins a tie.
// Rows whose candidates do not fit in LDS (heavy ties) take a fallback that
// runs the same radix select straight over the row in global memory.
// Integer histograms make every path deterministic.
#include "li_internal.h"
#include "li_select.h"

namespace li {
namespace {

constexpr int kFin = 1024;  // threads of the final kernel
constexpr int kFinWaves = kFin / 64;
constexpr int kCap = 12288;  // candidates held in LDS
constexpr int kCol = 256;    // threads of the collect kernel

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

// One radix level over `count` keys: histogram of the `nb` digits at `shift`
// among the keys matching (prefix, pmask), then the digit that holds the
// `remaining`-th largest.  Leaves {digit, #keys above it} in sh[1], sh[2].
template <typename KeyAt>
__device__ void radix_level(KeyAt key_at, int64_t count, uint32_t prefix, uint32_t pmask, int shift,
                            uint32_t nb, uint32_t remaining, uint32_t* hist, uint32_t* wsum,
                            int32_t* sh) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kSelBins; i += kFin) hist[i] = 0;
  if (tid == 0) {
    sh[1] = 0;
    sh[2] = 0;
  }
  __syncthreads();
  for (int64_t i = tid; i < count; i += kFin) {
    const uint32_t key = key_at(i);
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  // Digits in descending order: thread t owns nb-1-2t and nb-2-2t (nb = 2048)
  // or nb-1-t (nb = 1024).
  const int per = (int)nb / kFin;
  uint32_t hhi, hlo = 0;
  int dhi, dlo = -1;
  if (per == 2) {
    dhi = (int)nb - 1 - 2 * tid;
    dlo = dhi - 1;
    hhi = hist[dhi];
    hlo = hist[dlo];
  } else {
    dhi = (int)nb - 1 - tid;
    hhi = hist[dhi];
  }
  uint32_t total;
  const uint32_t above = block_excl_scan<kFin>(hhi + hlo, wsum, total);
  if (above < remaining && above + hhi >= remaining) {
    sh[1] = dhi;
    sh[2] = (int32_t)above;
  } else if (dlo >= 0 && above + hhi < remaining && above + hhi + hlo >= remaining) {
    sh[1] = dlo;
    sh[2] = (int32_t)(above + hhi);
  }
  __syncthreads();
}

// Ordered compaction over `count` candidates in position order: keep keys > T
// and the first m keys equal to T, writing slot = #gt-before + min(#eq-before, m).
template <typename KeyAt, typename PosAt>
__device__ void compact(const Row& row, KeyAt key_at, PosAt pos_at, int64_t count, uint32_t T,
                        uint32_t m, int64_t kk, uint32_t* wsum) {
  const int tid = threadIdx.x;
  uint32_t gt_run = 0, eq_run = 0;
#pragma unroll 1
  for (int64_t base = 0; base < count; base += 4 * kFin) {
    const int64_t i0 = base + 4 * tid;
    uint32_t fl[4];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fl[e] = 0;
      if (i0 + e < count) {
        const uint32_t key = key_at(i0 + e);
        fl[e] = key > T ? 2u : (key == T ? 1u : 0u);
      }
      cg += fl[e] >> 1;
      ce += fl[e] & 1u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<kFin>((cg << 16) | ce, wsum, total);
    uint32_t gb = gt_run + (ex >> 16), eb = eq_run + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (fl[e] == 2u) {
        const int64_t slot = (int64_t)gb + (eb < m ? eb : m);
        if (slot < kk) row.out[slot] = map_pos(row, pos_at(i0 + e));
        ++gb;
      } else if (fl[e] == 1u) {
        const int64_t slot = (int64_t)gb + eb;
        if (eb < m && slot < kk) row.out[slot] = map_pos(row, pos_at(i0 + e));
        ++eb;
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
  }
}

// Full radix select over keys read through key_at (3 levels of 11/11/10 bits
// starting from a known level-0 digit when `levels_from` = 1), then the
// ordered compaction.  Used both on LDS candidates and, as the fallback, on a
// row in global memory.
template <typename KeyAt, typename PosAt>
__device__ void select_keys(const Row& row, KeyAt key_at, PosAt pos_at, int64_t count,
                            uint32_t prefix, uint32_t pmask, uint32_t remaining, int first_level,
                            int64_t kk, uint32_t* hist, uint32_t* wsum, int32_t* sh) {
#pragma unroll 1
  for (int level = first_level; level < 3; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const uint32_t nb = level == 2 ? 1024u : 2048u;
    radix_level(key_at, count, prefix, pmask, shift, nb, remaining, hist, wsum, sh);
    prefix |= (uint32_t)sh[1] << shift;
    pmask |= (nb - 1) << shift;
    remaining -= (uint32_t)sh[2];
    __syncthreads();
  }
  compact(row, key_at, pos_at, count, prefix, remaining, kk, wsum);
}

enum SelHow : int32_t { kSelPre = 0, kSelSelf = 1, kSelFull = 2 };

__global__ __launch_bounds__(kFin) void topk_final_kernel(TopkRows a, SelWs ws, int how) {
  __shared__ uint2 cand[kCap];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t segoff[kFin];
  __shared__ uint32_t wsum[kFinWaves];
  __shared__ int32_t sh[4];
  __shared__ uint32_t shb[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const Row row = get_row(a, r, sh);
  const int64_t n = row.n;
  const int k = a.k;
  const int64_t kk = n < k ? n : (int64_t)k;

  if (kk == n) {  // everything visible is kept
    for (int64_t i = tid; i < k; i += kFin) row.out[i] = (i < n) ? map_pos(row, i) : -1;
    return;
  }
  for (int64_t i = kk + tid; i < k; i += kFin) row.out[i] = -1;

  auto gkey = [&](int64_t i) { return score_key(row.p[i]); };
  auto gpos = [&](int64_t i) { return i; };

  uint32_t bstar, above, eq;
  if (how == kSelFull) {
    for (int i = tid; i < kSelBins; i += kFin) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kFin) atomicAdd(&hist[gkey(i) >> kSelShift], 1u);
    __syncthreads();
    block_find_bin<kFin>([&](int b) { return hist[b]; }, (uint32_t)kk, wsum, shb);
    bstar = shb[0];
    above = shb[1];
    eq = shb[2];
  } else if (how == kSelPre) {
    const uint32_t* gh = ws.ghist + (int64_t)r * kSelBins;
    block_find_bin<kFin>([&](int b) { return gh[b]; }, (uint32_t)kk, wsum, shb);
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
  if (nc > kCap || above >= (uint32_t)kk) {
    // Fallback: radix select straight over the row in global memory.
    select_keys(row, gkey, gpos, n, 0u, 0u, (uint32_t)kk, 0, kk, hist, wsum, sh);
    return;
  }

  if (how == kSelPre) {
    // Segment offsets (one thread per segment), then every candidate is copied
    // independently: candidate i belongs to the last segment starting at or before i.
    int64_t nseg_row = (n + kSeg - 1) / kSeg;
    nseg_row = nseg_row < ws.nseg ? nseg_row : ws.nseg;
    nseg_row = nseg_row < kFin ? nseg_row : kFin;
    const uint32_t c = tid < nseg_row ? ws.cnt[(int64_t)r * ws.nseg + tid] : 0u;
    uint32_t total;
    const uint32_t o = block_excl_scan<kFin>(c, wsum, total);
    if (tid < nseg_row) segoff[tid] = o;
    __syncthreads();
    const int64_t ncp = (int64_t)total < nc ? (int64_t)total : nc;
    for (int64_t i = tid; i < ncp; i += kFin) {
      int lo = 0, hi = (int)nseg_row - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segoff[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
      }
      cand[i] = ws.cand[((int64_t)r * ws.nseg + lo) * kSeg + (i - segoff[lo])];
    }
  } else {
    // Ordered collection of the keys whose level-0 bin is >= b*.
    uint32_t run = 0;
#pragma unroll 1
    for (int64_t base = 0; base < n; base += 4 * kFin) {
      const int64_t i0 = base + 4 * tid;
      uint32_t key[4];
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = (i0 + e < n) ? gkey(i0 + e) : 0u;
        c += (i0 + e < n && (key[e] >> kSelShift) >= bstar) ? 1u : 0u;
      }
      uint32_t total;
      uint32_t pos = run + block_excl_scan<kFin>(c, wsum, total);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i0 + e < n && (key[e] >> kSelShift) >= bstar) {
          if (pos < (uint32_t)kCap) cand[pos] = make_uint2(key[e], (uint32_t)(i0 + e));
          ++pos;
        }
      }
      run += total;
    }
  }
  __syncthreads();
  auto lkey = [&](int64_t i) { return cand[i].x; };
  auto lpos = [&](int64_t i) { return (int64_t)cand[i].y; };
  select_keys(row, lkey, lpos, nc, bstar << kSelShift, 0xFFE00000u, (uint32_t)kk - above, 1, kk, hist,
              wsum, sh);
}

// One workgroup per (segment, row): the segment's candidates, in position
// order.  Each thread owns 32 consecutive positions, so all loads are issued
// before the single block scan.
constexpr int kColPer = kSeg / kCol;

__global__ __launch_bounds__(kCol) void topk_collect_kernel(TopkRows a, SelWs ws) {
  __shared__ uint32_t wsum[kCol / 64];
  __shared__ int32_t sh[4];
  __shared__ uint32_t shb[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.y, s = blockIdx.x;
  const Row row = get_row(a, r, sh);
  const int64_t n = row.n;
  if (n <= a.k) return;
  const int64_t s0 = (int64_t)s * kSeg;
  if (s0 >= n) return;
  const int64_t s1 = (s0 + kSeg) < n ? (s0 + kSeg) : n;
  const uint32_t* gh = ws.ghist + (int64_t)r * kSelBins;
  block_find_bin<kCol>([&](int b) { return gh[b]; }, (uint32_t)a.k, wsum, shb);
  const uint32_t bstar = shb[0];
  const int64_t i0 = s0 + (int64_t)kColPer * tid;
  uint32_t key[kColPer];
  uint32_t flags = 0, c = 0;
#pragma unroll
  for (int e = 0; e < kColPer; ++e) {
    const bool in = i0 + e < s1;
    key[e] = in ? score_key(row.p[i0 + e]) : 0u;
    const uint32_t f = (in && (key[e] >> kSelShift) >= bstar) ? 1u : 0u;
    flags |= f << e;
    c += f;
  }
  uint32_t total;
  uint32_t pos = block_excl_scan<kCol>(c, wsum, total);
  uint2* dst = ws.cand + ((int64_t)r * ws.nseg + s) * kSeg;
#pragma unroll
  for (int e = 0; e < kColPer; ++e) {
    if ((flags >> e) & 1u) {
      dst[pos] = make_uint2(key[e], (uint32_t)(i0 + e));
      ++pos;
    }
  }
  if (tid == 0) ws.cnt[(int64_t)r * ws.nseg + s] = total;
}

// Sums the scan workgroups' 16-bit partial histograms of each row:
// one workgroup per (256-bin slice, row).
__global__ __launch_bounds__(256) void hist_reduce_kernel(TopkRows a, SelWs ws) {
  __shared__ int32_t sh[4];
  const int r = blockIdx.y;
  const Row row = get_row(a, r, sh);
  if (row.n <= a.k) return;
  int64_t nw = (row.n + ws.chunk - 1) / ws.chunk;
  nw = nw < ws.nwg ? nw : ws.nwg;
  const int bin = blockIdx.x * 256 + threadIdx.x;
  const uint16_t* p = ws.part + (int64_t)r * ws.nwg * kSelBins + bin;
  uint32_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  int64_t w = 0;
  for (; w + 4 <= nw; w += 4) {
    s0 += p[(w + 0) * kSelBins];
    s1 += p[(w + 1) * kSelBins];
    s2 += p[(w + 2) * kSelBins];
    s3 += p[(w + 3) * kSelBins];
  }
  for (; w < nw; ++w) s0 += p[w * kSelBins];
  ws.ghist[(int64_t)r * kSelBins + bin] = s0 + s1 + s2 + s3;
}

}  // namespace

hipError_t launch_hist_reduce(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  hist_reduce_kernel<<<dim3(kSelBins / 256, (unsigned)a.rows), dim3(256), 0, stream>>>(a, ws);
  return hipGetLastError();
}

hipError_t launch_topk_collect(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  if (a.rows <= 0 || ws.nseg <= 0) return hipSuccess;
  topk_collect_kernel<<<dim3((unsigned)ws.nseg, (unsigned)a.rows), dim3(kCol), 0, stream>>>(a, ws);
  return hipGetLastError();
}

hipError_t launch_topk_pre(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  topk_final_kernel<<<dim3((unsigned)a.rows), dim3(kFin), 0, stream>>>(a, ws, kSelPre);
  return hipGetLastError();
}

hipError_t launch_topk_self(const TopkRows& a, const SelWs& ws, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  topk_final_kernel<<<dim3((unsigned)a.rows), dim3(kFin), 0, stream>>>(a, ws, kSelSelf);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkRows& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  SelWs none = {};
  topk_final_kernel<<<dim3((unsigned)a.rows), dim3(kFin), 0, stream>>>(a, none, kSelFull);
  return hipGetLastError();
}

}  // namespace li
