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
  // Bucket mode (bucket = 1): part holds each scan workgroup's descending
  // prefix counts (part[b] = its keys in bins >= b) and blist [rows][nwg][chunk]
  // its keys at or above its own k-th largest bin as (key, position) pairs in
  // descending bin order, so the keys in bins >= b are the first part[b].
  uint2* blist;
  int32_t bucket;
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

// Buffer resource word 3 for gfx9 parts (32-bit data format, raw addressing)
// and an offset past the end of any resource: a buffer store there is dropped
// by the range check, so a masked store needs no branch.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kBufferDrop = 0x80000000u;

// End of a scan workgroup in bucket mode.  lhist holds the level-0 counts of
// the workgroup's n keys (sk[0 .. n-1], score_key of the scores, positions
// pos0 + i) followed by 128 spare words; NT threads, PER = 8 bins each.
// Stores the descending prefix counts to pdst (16-bit: n <= CH <= 65535), then
// writes every key whose bin is at or above the bin of the workgroup's own
// min(k, n)-th largest key to ldst, bin by bin from the top (a key of a lower
// bin cannot be among the row's k largest: the k-th largest of a part of the
// row is at most the k-th largest of the row).  The order inside a bin is that
// of the LDS cursor atomics; the selection does not depend on it.  lhist and
// sk are overwritten (cursors; the list is staged over the keys when it
// fits); sh holds two words of scratch.
template <int NT, int CH>
__device__ __forceinline__ void bucket_epilogue(uint32_t* lhist, uint32_t* sk, int n, int k, uint32_t pos0,
                                                uint16_t* pdst, uint2* ldst, uint32_t* wsum, uint32_t* sh) {
  constexpr int PER = kSelBins / NT;
  static_assert(PER == 8 && CH % (4 * NT) == 0 && CH < 65536, "eight bins (one 16-byte partial store) per thread");
  const int t = threadIdx.x;
  uint32_t h[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    h[i] = lhist[kSelBins - 1 - (t * PER + i)];
    sum += h[i];
  }
  uint32_t total;
  uint32_t run = block_excl_scan<NT>(sum, wsum, total);  // keys in the bins above this thread's
  const uint32_t kk = (uint32_t)(k < n ? k : n);
  uint32_t pv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bin = kSelBins - 1 - (t * PER + i);
    const uint32_t above = run;
    run += h[i];
    pv[i] = run;
    lhist[bin] = above;  // first slot of the bin's keys
    if (above < kk && run >= kk) {
      sh[0] = (uint32_t)bin;  // the floor bin
      sh[1] = run;            // keys written
    }
  }
  // bins 2040 - 8t .. 2047 - 8t in ascending order
  const i32x4 pk = {(int)(pv[7] | (pv[6] << 16)), (int)(pv[5] | (pv[4] << 16)), (int)(pv[3] | (pv[2] << 16)),
                    (int)(pv[1] | (pv[0] << 16))};
  *reinterpret_cast<i32x4*>(pdst + (kSelBins - PER) - PER * t) = pk;
  __syncthreads();
  const uint32_t f = sh[0], nkeep = sh[1];
  // Thread t takes keys 4t .. 4t+3 of each 4*NT (16-byte LDS reads).
  constexpr int R4 = CH / (4 * NT);
  uint32_t key[4 * R4], slot[4 * R4];
#pragma unroll
  for (int j = 0; j < R4; ++j) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(&sk[4 * (t + NT * j)]);
    key[4 * j] = (uint32_t)v.x;
    key[4 * j + 1] = (uint32_t)v.y;
    key[4 * j + 2] = (uint32_t)v.z;
    key[4 * j + 3] = (uint32_t)v.w;
  }
  auto idx = [&](int e) { return 4 * (t + NT * (e >> 2)) + (e & 3); };
  auto keep = [&](int e) { return idx(e) < n && (key[e] >> kSelShift) >= f; };
  // Every cursor update is issued before any result is used; a lane with
  // nothing to place adds 0 to a spare word of its own (no branch).
  const int lane = t & 63;
#pragma unroll
  for (int e = 0; e < 4 * R4; ++e) {
    const bool kp = keep(e);
    slot[e] = atomicAdd(&lhist[kp ? (int)(key[e] >> kSelShift) : kSelBins + lane], kp ? 1u : 0u);
  }
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  constexpr int kStage = CH / 2;  // pairs that fit where the keys were
  if (nkeep <= (uint32_t)kStage) {
    // Staged in LDS over the keys (all read above), then written out with
    // 16-byte stores.  A lane with nothing to stage writes a spare pair.
    __syncthreads();
    u32x2* stage = reinterpret_cast<u32x2*>(sk);
    u32x2* spare = reinterpret_cast<u32x2*>(lhist + kSelBins) + lane;
#pragma unroll
    for (int e = 0; e < 4 * R4; ++e) {
      const bool kp = keep(e);
      *(kp ? stage + slot[e] : spare) = u32x2{key[e], pos0 + (uint32_t)idx(e)};
    }
    __syncthreads();
    const i32x4* src = reinterpret_cast<const i32x4*>(sk);
    i32x4* dst = reinterpret_cast<i32x4*>(ldst);
    for (uint32_t i = (uint32_t)t; 2 * i < nkeep; i += NT) {
      if (2 * i + 1 < nkeep) {
        dst[i] = src[i];
      } else {
        const i32x4 v = src[i];
        ldst[2 * i] = make_uint2((uint32_t)v.x, (uint32_t)v.y);
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ldst, (short)0, 8 * n, kBufferWord3);
#pragma unroll
    for (int e = 0; e < 4 * R4; ++e)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{key[e], pos0 + (uint32_t)idx(e)}, rs,
                                            keep(e) ? 8u * slot[e] : kBufferDrop, 0, 0);
  }
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
