// Per-row top-k selection on gfx950 (the step that turns indexer scores into
// the index tensor: "IndexCache: Cross-Layer Index Reuse for Sparse
// Attention", Deep Dive, the F layer takes top-k of its scores).
//
// One workgroup of 1024 threads owns one row.  Scores are mapped to
// order-preserving uint32 keys (-0 folded onto +0).  A radix select over the
// key bits (11 + 11 + 10, one LDS histogram per level, integer atomics so the
// result is deterministic) finds the exact k-th largest key T and the number
// m of elements equal to T that still fit.  A last pass walks the row in
// position order: a block-wide scan of the packed counts (#greater, #equal)
// gives every kept element its output slot,
//   slot = #greater-before + min(#equal-before, m),
// so the output comes out in ascending position order and, among elements
// equal to T, the lower positions win.  Rows with at most k visible elements
// return all of them; unused slots are -1.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkBins = 2048;

// Exclusive block-wide scan of one uint32 per thread; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    const uint32_t s = wsum[i];
    before += (i < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();  // wsum may be reused by the next call
  total = tot;
  return before + inc - v;
}

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
  return row;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkRows a) {
  __shared__ uint32_t hist[kTkBins];
  __shared__ uint32_t wsum[kTkWaves];
  __shared__ int32_t sh[4];
  const int tid = threadIdx.x;
  const Row row = get_row(a, blockIdx.x, sh);
  const int64_t n = row.n > 0 ? row.n : 0;
  const int k = a.k;
  const int64_t kk = n < k ? n : (int64_t)k;

  if (kk == n) {  // everything visible is kept
    for (int64_t i = tid; i < k; i += kTkThreads)
      row.out[i] = (i < n) ? (row.map ? row.map[i] : (int32_t)i) : -1;
    return;
  }

  // ---- radix select of the kk-th largest key --------------------------------
  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)kk;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const uint32_t nb = level == 2 ? 1024u : 2048u;
    for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0;
    if (tid == 0) {
      sh[1] = 0;
      sh[2] = 0;
    }
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTkThreads) {
      const uint32_t key = score_key(row.p[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // Bins in descending order: thread t owns the two bins nb-1-2t and nb-2-2t
    // (level 2: one bin, nb-1-t, for t < 1024).
    const int per = (int)nb / kTkThreads;
    uint32_t hhi = 0, hlo = 0;
    int dhi = -1, dlo = -1;
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
    const uint32_t above = block_excl_scan(hhi + hlo, wsum, total);
    if (above < remaining && above + hhi >= remaining) {
      sh[1] = dhi;
      sh[2] = (int32_t)above;
    } else if (dlo >= 0 && above + hhi < remaining && above + hhi + hlo >= remaining) {
      sh[1] = dlo;
      sh[2] = (int32_t)(above + hhi);
    }
    __syncthreads();
    prefix |= (uint32_t)sh[1] << shift;
    pmask |= (nb - 1) << shift;
    remaining -= (uint32_t)sh[2];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t m = remaining;  // elements equal to T to keep, lowest positions first

  // ---- ordered compaction ----------------------------------------------------
  uint32_t gt_run = 0, eq_run = 0;
#pragma unroll 1
  for (int64_t base = 0; base < n; base += 4 * kTkThreads) {
    const int64_t i0 = base + 4 * tid;
    uint32_t fl[4];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fl[e] = 0;
      if (i0 + e < n) {
        const uint32_t key = score_key(row.p[i0 + e]);
        fl[e] = key > T ? 2u : (key == T ? 1u : 0u);
      }
      cg += fl[e] >> 1;
      ce += fl[e] & 1u;
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan((cg << 16) | ce, wsum, total);
    uint32_t gb = gt_run + (ex >> 16), eb = eq_run + (ex & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + e;
      if (fl[e] == 2u) {
        const int64_t slot = (int64_t)gb + (eb < m ? eb : m);
        if (slot < kk) row.out[slot] = row.map ? row.map[i] : (int32_t)i;
        ++gb;
      } else if (fl[e] == 1u) {
        const int64_t slot = (int64_t)gb + eb;
        if (eb < m && slot < kk) row.out[slot] = row.map ? row.map[i] : (int32_t)i;
        ++eb;
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xFFFFu;
  }
  for (int64_t i = kk + tid; i < k; i += kTkThreads) row.out[i] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkRows& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  topk_kernel<<<dim3((unsigned)a.rows), dim3(kTkThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace li
