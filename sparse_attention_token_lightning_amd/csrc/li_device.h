// Device-side helpers shared by the gfx950 kernels of the lightning-indexer
// library: MFMA operand vector types, exact fp8/bf16 -> MFMA-operand
// conversions, the order-preserving key used by the top-k selection, and
// wavefront (64-lane) scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kWave = 64;

// Index of the calling wavefront in its workgroup, as a wave-uniform (scalar)
// value: the compiler cannot prove threadIdx.x >> 6 is uniform, and loops
// bounded by values derived from it would otherwise run under an exec mask,
// with conservative waits for every outstanding load.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// 16-byte global load / store through a plain vector type.
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }

// Loads of data a call streams once (key cache, latent cache and their
// scales): non-temporal, so the lines are not kept for reuse in the caches.
// A plain 553 MB read stream with the decode scan's pattern runs at about
// 6.1 TB/s with ordinary loads and 7.0 TB/s with these.
__device__ __forceinline__ i32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}
__device__ __forceinline__ i32x2 ld8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(p));
}
__device__ __forceinline__ float ldf_stream(const float* p) { return __builtin_nontemporal_load(p); }

// Raw buffer resource over `bytes` bytes from p (stride 0, 32-bit data
// format word of the gfx9 family).  A buffer load whose per-lane offset
// (register offset + instruction offset) is at or past `bytes` returns zeros
// and touches no memory, so loads near the end of a range need no clamp, and
// their offsets are 32-bit with the constant part in the instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// 16-byte buffer load with the non-temporal hint (cache-policy bit NT); a
// constant added to voff lands in the instruction's offset field.
__device__ __forceinline__ i32x4 buf_ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2);
}


// Four OCP E4M3FN bytes (one dword, byte 0 first) -> four bf16, exact: every
// E4M3FN value, subnormals included, is a bf16 normal number.  Uses gfx950's
// packed fp8 -> bf16 conversion with a unit scale.
__device__ __forceinline__ i32x2 fp8x4_to_bf16x4(int v) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  i32x2 r;
  r.x = __builtin_bit_cast(int, lo);
  r.y = __builtin_bit_cast(int, hi);
  return r;
}

// Eight fp8 bytes (two dwords) -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(int a, int b) {
  i32x2 x = fp8x4_to_bf16x4(a), y = fp8x4_to_bf16x4(b);
  i32x4 r = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(bf16x8, r);
}

// One fp8 byte (OCP E4M3FN) -> float, exact.
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  const int v = (int)(byte & 0xFFu);
  return __builtin_bit_cast(float, fp8x4_to_bf16x4(v).x << 16);
}

// 32x32x64 fp8 x fp8 -> fp32 matrix product (E4M3 operands, unit scales).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x128 fp8 x fp8 -> fp32 matrix product (E4M3 operands, unit scales).
// Operand lane l holds row / column (l & 15) and 32 consecutive K bytes of
// lane group l >> 4 (A and B pair K the same way); result lane l holds rows
// 4 * (l >> 4) + i, column l & 15.
__device__ __forceinline__ f32x4 mfma_fp8_16(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Cross-lane folds with gfx950's lane-swap instructions.  swap_sum32(a, b):
// lanes 0-31 get a[l] + a[l + 32], lanes 32-63 get b[l - 32] + b[l].
// swap_sum16(a, b): in each 32-lane half, lanes 0-15 get a[l] + a[l + 16] and
// lanes 16-31 get b[l - 16] + b[l].  The swap returns both registers; the
// empty asm keeps the second one a distinct value (without it this compiler
// folds first + second into first + first).
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false);
  unsigned x = sw[0], y = sw[1];
  asm volatile("" : "+v"(y));
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false);
  unsigned x = sw[0], y = sw[1];
  asm volatile("" : "+v"(y));
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Two bf16 (one dword) -> two fp16.  Exact for |x| in [2^-17, 65504]: bf16
// carries 8 significant bits, fp16 11 (subnormals down to 2^-24).
__device__ __forceinline__ int bf16x2_to_f16x2(int v) {
  float lo = __builtin_bit_cast(float, v << 16);
  float hi = __builtin_bit_cast(float, v & (int)0xFFFF0000u);
  f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  return __builtin_bit_cast(int, h);
}

__device__ __forceinline__ i32x4 bf16x8_to_f16x8(i32x4 v) {
  i32x4 r = {bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z),
             bf16x2_to_f16x2(v.w)};
  return r;
}

// ReLU on the bit pattern: a float with the sign bit set (negative, or -0) is
// a negative int32, so max(int, 0) yields +0 for it and leaves positive
// floats unchanged.  One integer op, with none of the NaN canonicalisation an
// IEEE float max needs.
__device__ __forceinline__ float relu(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Order-preserving map from an fp32 score to a uint32 key: a larger score
// gives a larger key, and -0 maps to the key of +0 so that the two compare
// equal (the tie then goes to the lower position).  NaN is not expected.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of a key (the inverse of score_key; -0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Sum of v over lanes l and l^32, in every lane.  (A cross-lane shuffle;
// gfx950's v_permlane32_swap would avoid the LDS crossbar, but this compiler
// folds the two results of that builtin into one register.)
__device__ __forceinline__ float sum_halves(float v) { return v + __shfl_xor(v, 32, 64); }

// Inclusive scan of a uint32 over the 64 lanes of a wavefront (every lane
// active), with DPP moves instead of LDS-crossbar shuffles: within each row
// of 16 lanes by row_shr 1, 2, 4 and 8 (a lane whose source lies outside its
// row adds the 0 it keeps), then lane 15 of rows 0 and 2 into rows 1 and 3
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return (uint32_t)x;
}

// Issue priority by progress: 3 in the first quarter of a wave's steps down
// to 0 in the last.  Two workgroups share each CU in the streaming scans, and
// the older one's waves would otherwise win every issue tie and finish well
// before the other's.
__device__ __forceinline__ void set_progress_priority(int step, int nsteps) {
  const int qtr = (4 * step) / (nsteps > 0 ? nsteps : 1);
  if (qtr == 0) __builtin_amdgcn_s_setprio(3);
  else if (qtr == 1) __builtin_amdgcn_s_setprio(2);
  else if (qtr == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

}  // namespace li
