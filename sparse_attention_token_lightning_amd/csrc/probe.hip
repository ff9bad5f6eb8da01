// Measurement aids, not part of the computation.
//
// Read-bandwidth probe:
// Streams a buffer once with the access pattern of the decode scan's key
// loads (16-byte non-temporal loads, each wave covering 1 KB contiguous per
// load, eight loads in flight per lane, a grid of 2048 four-wave workgroups
// striding over the buffer) and does nothing with the data but fold it into one word per
// wave, so the loads cannot be dropped.  Its duration gives the read rate
// this GPU reaches for such a stream, the practical ceiling that the
// HBM-bound kernels are compared against next to the published peak.
//
// Matrix-core rate probe: every wave of a grid that fills the GPU (eight
// waves per SIMD) runs two independent accumulator chains of one of the
// product forms the scans use, over eight A and eight B operand registers.
// The operands hold either one repeated value (1.0) or pseudo-random values
// with random signs and mantissas.  Each workgroup records how many shader
// clock cycles and how many 100 MHz real-time ticks it ran, so the host gets
// both the product rate and the shader clock it ran at.  The two operand
// kinds bracket the rate: the chip lowers its clock under the power drawn by
// products on varying data, so the random form is the ceiling that applies
// to a scan over real keys.
#include "../../include/li.h"
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeBlocks = 2048;
static_assert(kProbeBlocks * (kProbeThreads / 64) == LI_READ_PROBE_SINK_WORDS, "one sink word per wave");

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const i32x4* __restrict__ p, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t step = (int64_t)kProbeThreads * kProbeUnroll;
  int64_t i = (int64_t)blockIdx.x * step + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * step;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < n16; i += stride) {
    i32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = ld16_stream(p + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  for (int u = 0; u < kProbeUnroll; ++u) {
    const int64_t j = i + u * kProbeThreads;
    if (j < n16) {
      const i32x4 v = ld16_stream(p + j);
      acc ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

constexpr int kMfmaBlocks = 2048;
static_assert(kMfmaBlocks * (kProbeThreads / 64) == LI_MFMA_PROBE_SINK_WORDS, "one sink word per wave");
static_assert(2 * kMfmaBlocks == LI_MFMA_PROBE_CLOCK_WORDS, "two clock words per workgroup");
static_assert(LI_MFMA_PROBE_PRODUCTS_PER_ITER == 16, "two chains of eight products per iteration");

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// One operand word (two 16-bit values or four fp8 bytes) of form F: 1.0 in
// every element, or random signs and mantissas with exponents spanning 16
// octaves around 1 (fp16 / bf16) or any finite E4M3 code.
template <int F, bool RND>
__device__ __forceinline__ int probe_word(uint32_t seed) {
  if (F == LI_MFMA_PROBE_FP8) {
    if (!RND) return 0x38383838;
    uint32_t w = probe_hash(seed);
    // bytes whose low seven bits are all ones (NaN) become 0x77 / 0xF7
    const uint32_t nan = ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    return (int)(w ^ (nan >> 4));
  }
  if (!RND) return F == LI_MFMA_PROBE_F16 ? 0x3C003C00 : 0x3F803F80;
  uint32_t h[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t r = probe_hash(seed * 2u + (uint32_t)i);
    if (F == LI_MFMA_PROBE_F16)  // sign, exponent 7..22, 10 mantissa bits
      h[i] = (r & 0x83FFu) | ((7u + ((r >> 10) & 15u)) << 10);
    else  // bf16: sign, exponent 119..134, 7 mantissa bits
      h[i] = (r & 0x807Fu) | ((119u + ((r >> 7) & 15u)) << 7);
  }
  return (int)(h[0] | (h[1] << 16));
}

// F: product form; RND: random (true) or constant operands.
template <int F, bool RND>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float* __restrict__ sink,
                                                                   uint32_t* __restrict__ clk) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  constexpr int W = F == LI_MFMA_PROBE_FP8 ? 8 : 4;  // operand words per lane
  const uint32_t seed = (blockIdx.x * kProbeThreads + threadIdx.x) * 256u;
  int a[8][W], b[8][W];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int j = 0; j < W; ++j) {
      a[r][j] = probe_word<F, RND>(seed + r * W + j);
      b[r][j] = probe_word<F, RND>(seed + 128u + r * W + j);
    }
  float out;
  if constexpr (F == LI_MFMA_PROBE_BF16) {
    f32x16 c0v = {}, c1v = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const i32x4 av = {a[r][0], a[r][1], a[r][2], a[r][3]};
        const i32x4 aw = {a[(r + 4) & 7][0], a[(r + 4) & 7][1], a[(r + 4) & 7][2], a[(r + 4) & 7][3]};
        const i32x4 bv = {b[r][0], b[r][1], b[r][2], b[r][3]};
        c0v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                      c0v, 0, 0, 0);
        c1v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bv),
                                                      c1v, 0, 0, 0);
      }
    }
    out = c0v[0] + c1v[0];
  } else {
    f32x4 c0v = {}, c1v = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if constexpr (F == LI_MFMA_PROBE_F16) {
          const i32x4 av = {a[r][0], a[r][1], a[r][2], a[r][3]};
          const i32x4 aw = {a[(r + 4) & 7][0], a[(r + 4) & 7][1], a[(r + 4) & 7][2], a[(r + 4) & 7][3]};
          const i32x4 bv = {b[r][0], b[r][1], b[r][2], b[r][3]};
          c0v = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv),
                                                       c0v, 0, 0, 0);
          c1v = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aw), __builtin_bit_cast(f16x8, bv),
                                                       c1v, 0, 0, 0);
        } else {
          i32x8 av, aw, bv;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            av[j] = a[r][j];
            aw[j] = a[(r + 4) & 7][j];
            bv[j] = b[r][j];
          }
          c0v = mfma_fp8_16(av, bv, c0v);
          c1v = mfma_fp8_16(aw, bv, c1v);
        }
      }
    }
    out = c0v[0] + c1v[0];
  }
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = out;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = (uint32_t)(__builtin_amdgcn_s_memtime() - c0);
    clk[2 * blockIdx.x + 1] = (uint32_t)(__builtin_amdgcn_s_memrealtime() - t0);
  }
}

}  // namespace

namespace {

template <int F>
hipError_t launch_mfma_probe_form(bool random_operands, int iters, float* sink, uint32_t* clk, hipStream_t stream) {
  if (random_operands)
    return launch_kernel(mfma_probe_kernel<F, true>, dim3(kMfmaBlocks), dim3(kProbeThreads), 0u, stream, iters, sink,
                         clk);
  return launch_kernel(mfma_probe_kernel<F, false>, dim3(kMfmaBlocks), dim3(kProbeThreads), 0u, stream, iters, sink,
                       clk);
}

}  // namespace

hipError_t launch_mfma_probe(int form, bool random_operands, int iters, float* sink, uint32_t* clk,
                             hipStream_t stream) {
  if (form == LI_MFMA_PROBE_F16)
    return launch_mfma_probe_form<LI_MFMA_PROBE_F16>(random_operands, iters, sink, clk, stream);
  if (form == LI_MFMA_PROBE_BF16)
    return launch_mfma_probe_form<LI_MFMA_PROBE_BF16>(random_operands, iters, sink, clk, stream);
  return launch_mfma_probe_form<LI_MFMA_PROBE_FP8>(random_operands, iters, sink, clk, stream);
}

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  return launch_kernel(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0u, stream,
                       reinterpret_cast<const i32x4*>(p), bytes / 16, sink);
}

}  // namespace li
