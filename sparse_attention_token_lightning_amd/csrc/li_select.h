// Shared pieces of the selection step (top-k) used by the scan kernels, which
// build the first radix level while they write scores, and by the top-k
// kernels.  A score's order-preserving uint32 key is split as
//   bits 31..21 (level 0, 2048 bins) | 20..10 (level 1) | 9..0 (level 2).
#pragma once
#include "li_device.h"

namespace li {

constexpr int kSelBins = 2048;   // level-0 bins
constexpr int kSelShift = 21;    // key >> kSelShift = level-0 bin
constexpr int kSelCoarse = 64;   // coarse bins: 32 consecutive level-0 bins each
constexpr int kSelFine = kSelBins / kSelCoarse;
constexpr int kSeg = 8192;       // scores per collect segment (doubled for large grids)

// Per-row state that the scan kernels hand to the top-k kernels through the
// caller's workspace.
struct SelWs {
  uint16_t* part;   // [rows][nwg][kSelBins] per-workgroup level-0 histograms (scan kernels)
  uint16_t* cpart;  // [rows][nwg][kSelCoarse] the same, summed over 32 consecutive bins
  int32_t nwg;      // partial histograms per row (the scan grid's x extent)
  int32_t chunk;    // positions of a row covered by one scan workgroup
  uint32_t* thr;    // [rows][4] {threshold bin, #keys above it, #keys in it, valid} (prefill)
  uint32_t* cnt;    // [rows][nseg] candidates per segment
  uint2* cand;      // [rows][nseg][seg] (key, position) candidates in position order
  int32_t nseg;
  int32_t seg;      // scores per collect segment (kSeg or 2 * kSeg)
  uint32_t* done;   // [rows] finished-segment counters (zeroed by the scan kernel)
  int32_t cap;      // LDS candidates of the final selection in the segmented top-k
};

// Writes a workgroup's LDS histogram (one 32-bit counter per bin, counts <
// 65536) as 16-bit partials, two bins per 32-bit store, and its coarse
// partial.  NT threads.
template <int NT>
__device__ __forceinline__ void store_partial(const uint32_t* lhist, uint16_t* dst, uint16_t* cdst) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  for (int i = threadIdx.x; i < kSelBins / 2; i += NT) d[i] = lhist[2 * i] | (lhist[2 * i + 1] << 16);
  for (int c = threadIdx.x; c < kSelCoarse; c += NT) {
    uint32_t sum = 0;
    for (int i = 0; i < kSelFine; ++i) sum += lhist[c * kSelFine + i];
    cdst[c] = (uint16_t)sum;
  }
}

// The same for a histogram already packed two 16-bit bins per word (bin b in
// half b & 1 of word b >> 1).
template <int NT>
__device__ __forceinline__ void store_partial_packed(const uint32_t* lhist, uint16_t* dst, uint16_t* cdst) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  for (int i = threadIdx.x; i < kSelBins / 2; i += NT) d[i] = lhist[i];
  for (int c = threadIdx.x; c < kSelCoarse; c += NT) {
    uint32_t sum = 0;
    for (int i = 0; i < kSelFine / 2; ++i) {
      const uint32_t v = lhist[c * (kSelFine / 2) + i];
      sum += (v & 0xFFFFu) + (v >> 16);
    }
    cdst[c] = (uint16_t)sum;
  }
}

// Exclusive scan of one uint32 per thread over a block of NT threads (NT/64
// wavefronts); also returns the block total.  Contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = wsum[i];
    before += (i < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Given a level-0 histogram (read through `get(bin)`), find the bin that
// holds the kk-th largest key.  Thread t of the NT-thread block owns bins
// 2047 - t*PER ... downwards.  Writes {bin, #above, #in bin} to out[0..2]
// (shared memory) and returns after a barrier.
template <int NT, typename Get>
__device__ __forceinline__ void block_find_bin(Get get, uint32_t kk, uint32_t* wsum, uint32_t* out) {
  constexpr int PER = kSelBins / NT;
  uint32_t h[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    h[i] = get(kSelBins - 1 - ((int)threadIdx.x * PER + i));
    sum += h[i];
  }
  uint32_t total;
  uint32_t run = block_excl_scan<NT>(sum, wsum, total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < kk && run + h[i] >= kk) {
      out[0] = (uint32_t)(kSelBins - 1 - ((int)threadIdx.x * PER + i));
      out[1] = run;
      out[2] = h[i];
    }
    run += h[i];
  }
  __syncthreads();
}

}  // namespace li
