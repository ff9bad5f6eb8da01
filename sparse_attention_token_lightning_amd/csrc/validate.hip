// Opt-in checks of device inputs (the LI_DEBUG_VALIDATE environment variable).
//
// The entry points never read device memory on the host, so on the normal
// path the preconditions on device contents (monotone kv_off, positive finite
// scales, no NaN/Inf codes, ascending candidate rows) are the caller's to
// keep.  With LI_DEBUG_VALIDATE set, an entry point first runs these kernels
// over its inputs, waits for them and returns LI_E_VALUE naming a violation
// it found.  Each kernel is a grid-stride loop with no other synchronisation;
// a violation is recorded by a compare-and-swap on a small device-resident
// record (the first report to land wins, its element index alongside).
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

__device__ uint32_t g_bad[4];  // [0] check id (0 = none), [1..2] element index (lo, hi)

__device__ void report(uint32_t check, int64_t i) {
  if (atomicCAS(&g_bad[0], 0u, check) == 0u) {
    g_bad[1] = (uint32_t)(uint64_t)i;
    g_bad[2] = (uint32_t)((uint64_t)i >> 32);
  }
}

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t gtid() { return (int64_t)blockIdx.x * kThreads + threadIdx.x; }
__device__ __forceinline__ int64_t gstride() { return (int64_t)gridDim.x * kThreads; }

__global__ __launch_bounds__(kThreads) void offsets_kernel(const int64_t* off, int32_t B, int64_t n_tok,
                                                           int32_t max_len) {
  for (int64_t b = gtid(); b <= B; b += gstride()) {
    const int64_t v = off[b];
    if (v < 0 || v > n_tok) report(kBadOffsetRange, b);
    if (b < B) {
      const int64_t len = off[b + 1] - v;
      if (len < 0) report(kBadOffsetOrder, b);
      else if (len > max_len) report(kBadLength, b);
    }
  }
}

__global__ __launch_bounds__(kThreads) void scales_kernel(const float* p, int64_t n, uint32_t check) {
  for (int64_t i = gtid(); i < n; i += gstride()) {
    const float v = p[i];
    if (!(v > 0.0f) || !isfinite(v)) report(check, i);
  }
}

__global__ __launch_bounds__(kThreads) void f32_kernel(const float* p, int64_t n, uint32_t check) {
  for (int64_t i = gtid(); i < n; i += gstride())
    if (!isfinite(p[i])) report(check, i);
}

// bf16: exponent field all ones is Inf or NaN.
__global__ __launch_bounds__(kThreads) void bf16_kernel(const uint16_t* p, int64_t n, uint32_t check) {
  for (int64_t i = gtid(); i < n; i += gstride())
    if ((p[i] & 0x7F80u) == 0x7F80u) report(check, i);
}

// OCP E4M3FN: 0x7F and 0xFF are its only NaN codes (it has no infinities).
__global__ __launch_bounds__(kThreads) void fp8_kernel(const uint8_t* p, int64_t n, uint32_t check) {
  for (int64_t i = gtid(); i < n; i += gstride())
    if ((p[i] & 0x7Fu) == 0x7Fu) report(check, i);
}

// Scores handed to li_topk: +-Inf are valid (masked entries), NaN is not.
// Row r holds len[r] scores (clamped to [0, cols]) or, without len, cols.
__global__ __launch_bounds__(kThreads) void nan_rows_kernel(const float* p, int64_t stride, int32_t rows,
                                                            int64_t cols, const int32_t* len) {
  for (int64_t i = gtid(); i < (int64_t)rows * cols; i += gstride()) {
    const int64_t r = i / cols, c = i % cols;
    int64_t n = len ? (int64_t)len[r] : cols;
    n = n < 0 ? 0 : (n > cols ? cols : n);
    if (c < n) {
      const float v = p[r * stride + c];
      if (v != v) report(kBadScores, r * stride + c);
    }
  }
}

__global__ __launch_bounds__(kThreads) void row_len_kernel(const int32_t* len, int32_t rows, int64_t stride) {
  for (int64_t r = gtid(); r < rows; r += gstride())
    if (len[r] < 0 || len[r] > stride) report(kBadRowLen, r);
}

__global__ __launch_bounds__(kThreads) void dst_rows_kernel(const int64_t* dst, int32_t M, int64_t n_tok) {
  for (int64_t m = gtid(); m < M; m += gstride())
    if (dst[m] < 0 || dst[m] >= n_tok) report(kBadDstRow, m);
}

// Candidate rows: valid entries strictly ascending inside [0, L_b), then -1 only.
__global__ __launch_bounds__(kThreads) void cands_kernel(const int32_t* cand, int32_t B, int32_t C,
                                                         const int64_t* off) {
  for (int64_t i = gtid(); i < (int64_t)B * C; i += gstride()) {
    const int64_t b = i / C, j = i % C;
    const int64_t len = off[b + 1] - off[b];
    const int32_t v = cand[i];
    if (v < -1 || v >= len) report(kBadCandidate, i);
    else if (j > 0) {
      const int32_t u = cand[i - 1];
      if (u == -1 ? v != -1 : (v != -1 && v <= u)) report(kBadCandidateOrder, i);
    }
  }
}

// One latent element (value index i of a cache with Dc values per row): a
// NaN/Inf code, and for the fp16 product form a bf16 value beyond fp16's
// range; at the first value of each scale block, that block's scale (finite
// and positive, and for an fp8 latent in the fp16 form small enough that
// 448 * scale stays inside fp16's range).
__device__ void check_latent_elem(const void* latent, bool fp8, int64_t i, int32_t Dc, const float* c_scale,
                                  int32_t nblk, bool fp16_form) {
  if (fp8) {
    if ((reinterpret_cast<const uint8_t*>(latent)[i] & 0x7Fu) == 0x7Fu) report(kBadLatent, i);
  } else {
    const uint16_t v = reinterpret_cast<const uint16_t*>(latent)[i];
    if ((v & 0x7F80u) == 0x7F80u) report(kBadLatent, i);
    else if (fp16_form && fabsf(__builtin_bit_cast(float, (uint32_t)v << 16)) > 65504.0f)
      report(kBadLatentRange, i);
  }
  const int32_t blk = nblk == 1 ? Dc : 128;
  const int64_t row = i / Dc;
  const int32_t c = (int32_t)(i - row * Dc);
  if (c_scale && c % blk == 0) {
    const int64_t si = row * nblk + c / blk;
    const float sc = c_scale[si];
    if (!(sc > 0.0f) || !isfinite(sc)) report(kBadCScale, si);
    else if (fp8 && fp16_form && 448.0f * sc > 65504.0f) report(kBadCScaleRange, si);
  }
}

__global__ __launch_bounds__(kThreads) void latent_kernel(const void* latent, bool fp8, int64_t n_tok, int32_t Dc,
                                                          const float* c_scale, int32_t nblk, bool fp16_form) {
  for (int64_t i = gtid(); i < n_tok * Dc; i += gstride())
    check_latent_elem(latent, fp8, i, Dc, c_scale, nblk, fp16_form);
}

// The latent rows an HS call reads: kv_off[b] + cand[b][j] for the entries
// inside [0, L_b) (entries outside are reported by cands_kernel, and the
// caller runs this check only once those have passed).
__global__ __launch_bounds__(kThreads) void cand_latent_kernel(const int32_t* cand, int32_t B, int32_t C,
                                                               const int64_t* off, const void* latent, bool fp8,
                                                               int32_t Dc, const float* c_scale, int32_t nblk,
                                                               bool fp16_form) {
  for (int64_t i = gtid(); i < (int64_t)B * C * Dc; i += gstride()) {
    const int64_t bj = i / Dc, b = bj / C;
    const int32_t v = cand[bj];
    if (v < 0 || v >= off[b + 1] - off[b]) continue;
    check_latent_elem(latent, fp8, (off[b] + v) * Dc + (i - bj * Dc), Dc, c_scale, nblk, fp16_form);
  }
}

unsigned blocks_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (unsigned)(b < 1 ? 1 : (b > 2048 ? 2048 : b));
}

}  // namespace

hipError_t validate_begin(hipStream_t s) {
  static const uint32_t zero[4] = {0u, 0u, 0u, 0u};
  return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_bad), zero, sizeof zero, 0, hipMemcpyHostToDevice, s);
}

void validate_offsets(const int64_t* off, int32_t B, int64_t n_tok, int32_t max_len, hipStream_t s) {
  offsets_kernel<<<blocks_for((int64_t)B + 1), kThreads, 0, s>>>(off, B, n_tok, max_len);
}
void validate_scales(const float* p, int64_t n, uint32_t check, hipStream_t s) {
  if (p && n > 0) scales_kernel<<<blocks_for(n), kThreads, 0, s>>>(p, n, check);
}
void validate_f32(const float* p, int64_t n, uint32_t check, hipStream_t s) {
  if (p && n > 0) f32_kernel<<<blocks_for(n), kThreads, 0, s>>>(p, n, check);
}
void validate_bf16(const void* p, int64_t n, uint32_t check, hipStream_t s) {
  if (p && n > 0) bf16_kernel<<<blocks_for(n), kThreads, 0, s>>>((const uint16_t*)p, n, check);
}
void validate_fp8(const void* p, int64_t n, uint32_t check, hipStream_t s) {
  if (p && n > 0) fp8_kernel<<<blocks_for(n), kThreads, 0, s>>>((const uint8_t*)p, n, check);
}
void validate_latent(const void* latent, bool fp8, int64_t n_tok, int32_t Dc, const float* c_scale,
                     bool fp16_form, hipStream_t s) {
  const int32_t nblk = fp8 ? (Dc + 127) / 128 : 1;
  if (latent && n_tok > 0 && Dc > 0)
    latent_kernel<<<blocks_for(n_tok * Dc), kThreads, 0, s>>>(latent, fp8, n_tok, Dc, c_scale, nblk, fp16_form);
}
void validate_cand_latent(const int32_t* cand, int32_t B, int32_t C, const int64_t* off, const void* latent,
                          bool fp8, int32_t Dc, const float* c_scale, bool fp16_form, hipStream_t s) {
  const int32_t nblk = fp8 ? (Dc + 127) / 128 : 1;
  if (B > 0 && C > 0 && Dc > 0)
    cand_latent_kernel<<<blocks_for((int64_t)B * C * Dc), kThreads, 0, s>>>(cand, B, C, off, latent, fp8, Dc,
                                                                            c_scale, nblk, fp16_form);
}
void validate_cands(const int32_t* cand, int32_t B, int32_t C, const int64_t* off, hipStream_t s) {
  if (B > 0 && C > 0) cands_kernel<<<blocks_for((int64_t)B * C), kThreads, 0, s>>>(cand, B, C, off);
}

void validate_score_rows(const float* p, int64_t stride, int32_t rows, int32_t n, const int32_t* len,
                         hipStream_t s) {
  const int64_t cols = len ? stride : n;
  if (rows > 0 && cols > 0)
    nan_rows_kernel<<<blocks_for((int64_t)rows * cols), kThreads, 0, s>>>(p, stride, rows, cols, len);
}
void validate_row_len(const int32_t* len, int32_t rows, int64_t stride, hipStream_t s) {
  if (len && rows > 0) row_len_kernel<<<blocks_for(rows), kThreads, 0, s>>>(len, rows, stride);
}

void validate_dst_rows(const int64_t* dst, int32_t M, int64_t n_tok, hipStream_t s) {
  if (M > 0) dst_rows_kernel<<<blocks_for(M), kThreads, 0, s>>>(dst, M, n_tok);
}

hipError_t validate_end(hipStream_t s, uint32_t* check, int64_t* index) {
  uint32_t r[4] = {0u, 0u, 0u, 0u};
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyFromSymbolAsync(r, HIP_SYMBOL(g_bad), sizeof r, 0, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  *check = r[0];
  *index = (int64_t)(((uint64_t)r[2] << 32) | r[1]);
  return e;
}

const char* validate_name(uint32_t check) {
  switch (check) {
    case kBadOffsetRange: return "kv_off entry outside [0, n_tok]";
    case kBadOffsetOrder: return "kv_off decreases";
    case kBadLength: return "a request longer than max_len";
    case kBadKScale: return "k_scale not finite and positive";
    case kBadQScale: return "q_scale not finite and positive";
    case kBadCScale: return "c_scale not finite and positive";
    case kBadW: return "w not finite";
    case kBadQ: return "q holds a NaN/Inf code";
    case kBadKeys: return "k_cache holds a NaN/Inf code";
    case kBadLatent: return "latent holds a NaN/Inf code";
    case kBadWDec: return "w_dec holds a NaN/Inf code";
    case kBadCandidate: return "cand_idx entry outside [-1, L_b)";
    case kBadCandidateOrder: return "cand_idx row not ascending with -1 only at its end";
    case kBadScores: return "scores hold a NaN";
    case kBadRowLen: return "row_len entry outside [0, row_stride]";
    case kBadDstRow: return "dst_row entry outside [0, n_tok)";
    case kBadHidden: return "h holds a NaN/Inf code";
    case kBadWEnc: return "w_enc holds a NaN/Inf code";
    case kBadLatentRange: return "latent value beyond fp16 range (|c| > 65504) for LI_LATENT_FP16";
    case kBadCScaleRange: return "fp8 latent block scale above 65504 / 448 for LI_LATENT_FP16";
    default: return "unknown check";
  }
}

}  // namespace li
