// C-ABI entry points of the lightning-indexer library (declared in li.h):
// argument validation, workspace carving and kernel dispatch.  Every check
// that can fail happens before the first launch; calls only enqueue work on
// the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/li.h"
#include "li_internal.h"

namespace {

thread_local std::string g_err;

// Opt-in measurement trace (li_trace_events): caller-created hipEvents that the
// entry points attach, two per kernel (start, stop), to their kernel launches.
thread_local hipEvent_t* g_trace = nullptr;
thread_local int32_t g_trace_cap = 0;
thread_local int32_t g_trace_n = 0;

void trace_begin() { g_trace_n = 0; }

li_status fail(li_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

li_status hip_check(hipError_t e, const char* what, hipStream_t s) {
  (void)s;
  if (e == hipSuccess) return LI_OK;
  return fail(LI_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// LI_DEBUG_VALIDATE, read at every call.
bool validate_on() {
  const char* e = getenv("LI_DEBUG_VALIDATE");
  return e != nullptr && *e != '\0' && strcmp(e, "0") != 0;
}

// Enqueues the checks `enqueue` adds, waits for them and reports the first
// failed one as LI_E_VALUE.
template <typename F>
li_status run_validation(hipStream_t s, F enqueue) {
  hipError_t e = li::validate_begin(s);
  if (e != hipSuccess) return fail(LI_E_HIP, "validation: %s", hipGetErrorString(e));
  enqueue();
  uint32_t check = 0;
  int64_t index = 0;
  e = li::validate_end(s, &check, &index);
  if (e != hipSuccess) return fail(LI_E_HIP, "validation: %s", hipGetErrorString(e));
  if (check != 0)
    return fail(LI_E_VALUE, "LI_DEBUG_VALIDATE: %s (element %lld)", li::validate_name(check),
                (long long)index);
  return LI_OK;
}

constexpr size_t kAlign = 256;
constexpr int64_t kHistBins = li::kSelBins;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive aligned regions out of the caller's workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* ws) : base((char*)ws) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(bytes);
    return p;
  }
};

int64_t nseg_for(int64_t rows, int64_t max_len) {
  const int64_t seg = li::seg_len_for(rows, max_len);
  return (max_len + seg - 1) / seg;
}

// Selection state for `rows` rows: per-row thresholds; with `chunk` > 0 also
// the scan workgroups' partial histograms (ceil(max_len / chunk) per row) and
// either the bucket lists (bucket mode) or the summed histograms and the
// collect segments' candidates.
size_t sel_ws(int64_t rows, int64_t max_len, int64_t chunk, bool bucket) {
  size_t s = align_up((size_t)rows * 16);  // thr
  if (chunk > 0) {
    const int64_t nwg = (max_len + chunk - 1) / chunk;
    s += align_up((size_t)rows * nwg * kHistBins * 2);
    if (bucket) {
      s += align_up((size_t)rows * nwg * chunk * 8);
    } else {
      const int64_t nseg = nseg_for(rows, max_len), seg = li::seg_len_for(rows, max_len);
      s += align_up((size_t)rows * nwg * li::kSelCoarse * 2) + align_up((size_t)rows * 4);
      s += align_up((size_t)rows * nseg * 4) + align_up((size_t)rows * nseg * seg * 8);
    }
  }
  return s;
}

li::SelWs carve_sel(Carver& cv, int64_t rows, int64_t max_len, int64_t chunk, int32_t k, bool bucket) {
  li::SelWs w = {};
  w.thr = (uint32_t*)cv.take((size_t)rows * 16);
  if (chunk > 0) {
    const int64_t nwg = (max_len + chunk - 1) / chunk;
    w.part = (uint16_t*)cv.take((size_t)rows * nwg * kHistBins * 2);
    w.nwg = (int32_t)nwg;
    w.chunk = (int32_t)chunk;
    if (bucket) {
      w.blist = (uint2*)cv.take((size_t)rows * nwg * chunk * 8);
      w.bucket = 1;
    } else {
      const int64_t nseg = nseg_for(rows, max_len), seg = li::seg_len_for(rows, max_len);
      w.cpart = (uint16_t*)cv.take((size_t)rows * nwg * li::kSelCoarse * 2);
      w.done = (uint32_t*)cv.take((size_t)rows * 4);
      w.cnt = (uint32_t*)cv.take((size_t)rows * nseg * 4);
      w.cand = (uint2*)cv.take((size_t)rows * nseg * seg * 8);
      w.nseg = (int32_t)nseg;
      w.seg = (int32_t)seg;
      w.cap = li::seg_cap_for(k);
    }
  }
  return w;
}

// Decode selects in bucket mode when its rows fit it (see li::bucket_ok);
// then the scan writes no dense scores unless the caller wants them.
bool decode_bucket(int64_t n_tok, int32_t B, int32_t max_len, int32_t k) {
  const int64_t chunk = li::decode_chunk(n_tok, B);
  return max_len > 0 && li::bucket_ok((max_len + chunk - 1) / chunk, chunk, k, max_len);
}

size_t decode_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t k, bool scores_given) {
  const bool bucket = decode_bucket(n_tok, B, max_len, k);
  size_t s = 0;
  if (!scores_given && !bucket) s += align_up((size_t)n_tok * 4);
  const int64_t rows = B > 0 ? B : 0;
  s += sel_ws(rows, max_len > 0 ? max_len : 0, li::decode_chunk(n_tok, B), bucket);
  return s;
}

// The prefill's candidate lists are sized for the worst case (every visible
// key of a row), so they cannot overflow; rows use a fraction of them.
size_t prefill_ws(int32_t T, int32_t L, bool scores_given) {
  (void)scores_given;
  size_t s = 0;
  const size_t rows = T > 0 ? (size_t)T : 0;
  s += align_up(rows * (size_t)(L > 0 ? L : 0) * 8) + align_up(rows * 4);
  s += align_up(rows * li::kLinRows * 128) + align_up(rows * li::kLinRows * 4);
  s += sel_ws(T > 0 ? T : 0, 0, 0, false);
  return s;
}

size_t latent_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dc,
                 bool scores_given) {
  const size_t rows = (size_t)(B > 0 ? B : 0) * (G > 0 ? G : 0);
  // absorbed queries: room for the two bf16 parts of LI_LATENT_SPLIT_BF16
  size_t s = align_up(rows * H * Dc * 4) + align_up(rows * H * 4);
  if (!scores_given) s += align_up((size_t)G * (size_t)n_tok * 4);
  s += sel_ws((int64_t)rows, max_len > 0 ? max_len : 0, li::latent_chunk(n_tok), false);
  return s;
}

size_t hs_ws(int32_t B, int32_t C, int32_t Gf, int32_t H, int32_t Dc, bool scores_given) {
  const size_t rows = (size_t)B * Gf;
  size_t s = align_up(rows * H * Dc * 4) + align_up(rows * H * 4);
  if (!scores_given) s += align_up(rows * (size_t)C * 4);
  return s;
}

li_status check_k(int32_t k) {
  if (k <= 0) return fail(LI_E_SHAPE, "k must be >= 1 (got %d)", k);
  if (k > LI_MAX_K) return fail(LI_E_UNSUPPORTED, "k must be <= %d (got %d)", LI_MAX_K, k);
  return LI_OK;
}

li_status check_heads(int32_t H, int32_t D, const char* dname) {
  if (H <= 0 || D <= 0) return fail(LI_E_SHAPE, "H and %s must be positive (H=%d %s=%d)", dname, H, dname, D);
  if (H > 64) return fail(LI_E_UNSUPPORTED, "H must be <= 64 (got %d)", H);
  if (D != 128) return fail(LI_E_UNSUPPORTED, "%s must be 128 (got %d)", dname, D);
  return LI_OK;
}

// Fewest heads each approximate product form is accepted for.  The score bar
// is |S_gpu - S_exact| <= 2e-3 * sum_h |w_h x_h|; a form whose per-head error
// is relative to sum_d |q_d k_d| (not to |x_h|) meets it only when no single
// cancelling head dominates that sum.  Measured worst error / bar on N(0,1)
// inputs and on queries spread over 2^-9 .. 2^0 inside each head:
//  - prefill (fp8 MFMA): H = 1 fails (err ~ 1.0 * A), H = 2 fails on spread
//    queries (9.5e-3 * A); H = 8: 8.3e-5 (random), 4.8e-4 (spread).
//  - latent, fp16 absorbed query: H = 2 fails (1.7e-2 * A), H = 4 1.9e-3,
//    H = 8 6.6e-4, H = 16 4.1e-4, H = 64 1.5e-4.
//  - latent, split bf16 query: H = 1 fails (1.8e-2 * A), H = 2 1.3e-4.
// Latent widths with kernels: 128, 192 (128 + a 64-value block) and 256.
bool dc_ok(int32_t Dc) { return Dc == 128 || Dc == 192 || Dc == 256; }

constexpr int32_t kPrefillMinHeads = 8;
constexpr int32_t kLatentFp16MinHeads = 16;  // below: the split form runs instead (bf16 latent)
constexpr int32_t kLatentMinHeads = 2;

li_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(LI_E_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  if (need > 0 && ws == nullptr) return fail(LI_E_NULL, "workspace pointer is NULL");
  return LI_OK;
}

// Device scratch of li_index_decode_noalloc, for callers that cannot
// allocate: one array per GPU the library runs on, held until the process
// ends.  Host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kScratchBytes = LI_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device.
li_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LI_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LI_E_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(LI_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (!p) return fail(LI_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LI_OK;
}

}  // namespace

namespace li {
void trace_next(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (g_trace && g_trace_n + 2 <= g_trace_cap) {
    *start = g_trace[g_trace_n];
    *stop = g_trace[g_trace_n + 1];
    g_trace_n += 2;
  }
}
}  // namespace li

extern "C" {

const char* li_status_str(li_status s) {
  switch (s) {
    case LI_OK: return "LI_OK";
    case LI_E_NULL: return "LI_E_NULL";
    case LI_E_SHAPE: return "LI_E_SHAPE";
    case LI_E_DTYPE: return "LI_E_DTYPE";
    case LI_E_WORKSPACE: return "LI_E_WORKSPACE";
    case LI_E_UNSUPPORTED: return "LI_E_UNSUPPORTED";
    case LI_E_HIP: return "LI_E_HIP";
    case LI_E_VALUE: return "LI_E_VALUE";
    default: return "LI_E_UNKNOWN";
  }
}

const char* li_last_error(void) { return g_err.c_str(); }

void li_trace_events(void** events, int32_t capacity) {
  g_trace = capacity > 0 ? (hipEvent_t*)events : nullptr;
  g_trace_cap = (events && capacity > 0) ? capacity : 0;
  g_trace_n = 0;
}

int32_t li_trace_count(void) { return g_trace_n; }

li_status li_read_probe(const void* p, size_t bytes, uint32_t* sink, void* stream) {
  g_err.clear();
  if (!p || !sink) return fail(LI_E_NULL, "p and sink are required");
  if (bytes % 16 != 0 || ((uintptr_t)p & 15) != 0)
    return fail(LI_E_SHAPE, "p must be 16-byte aligned and bytes a multiple of 16");
  trace_begin();
  return hip_check(li::launch_read_probe(p, (int64_t)bytes, sink, (hipStream_t)stream), "read_probe launch",
                   (hipStream_t)stream);
}

li_status li_mfma_probe(int32_t form, int32_t random_operands, int32_t iters, float* sink, uint32_t* clk,
                        void* stream) {
  g_err.clear();
  if (!sink || !clk) return fail(LI_E_NULL, "sink and clk are required");
  if (form != LI_MFMA_PROBE_F16 && form != LI_MFMA_PROBE_BF16 && form != LI_MFMA_PROBE_FP8)
    return fail(LI_E_SHAPE, "form must be LI_MFMA_PROBE_F16, LI_MFMA_PROBE_BF16 or LI_MFMA_PROBE_FP8");
  if (iters < 1 || iters > (1 << 20)) return fail(LI_E_SHAPE, "iters must be in [1, 2^20]");
  trace_begin();
  return hip_check(li::launch_mfma_probe(form, random_operands != 0, iters, sink, clk, (hipStream_t)stream),
                   "mfma_probe launch", (hipStream_t)stream);
}


size_t li_index_decode_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t k,
                          int32_t has_out_scores) {
  (void)k;
  return decode_ws(B, n_tok, max_len, k, has_out_scores != 0);
}

// Host-side argument checks of a decode call (everything but the workspace).
static li_status check_decode_args(const void* q, li_dtype q_dt, const float* w, const void* k_cache,
                                   li_dtype k_dt, const int64_t* kv_off, int32_t B, int64_t n_tok, int32_t max_len,
                                   int32_t H, int32_t D, int32_t k, const int32_t* out_idx) {
  if (!q || !w || !k_cache || !kv_off || !out_idx)
    return fail(LI_E_NULL, "q, w, k_cache, kv_off and out_idx are required");
  if (q_dt != LI_BF16) return fail(LI_E_DTYPE, "decode q must be LI_BF16");
  if (k_dt != LI_BF16 && k_dt != LI_FP8_E4M3)
    return fail(LI_E_DTYPE, "decode k_cache must be LI_BF16 or LI_FP8_E4M3");
  if (B < 0 || n_tok < 0 || max_len < 0)
    return fail(LI_E_SHAPE, "B, n_tok and max_len must be >= 0");
  if (n_tok >= (int64_t)1 << 40) return fail(LI_E_UNSUPPORTED, "n_tok too large");
  // fp8 keys are read through 32-bit buffer offsets within a request
  if (k_dt == LI_FP8_E4M3 && max_len > li::kDecodeFp8MaxLen)
    return fail(LI_E_UNSUPPORTED, "fp8 decode: max_len above 33550336");
  li_status st;
  if ((st = check_k(k)) || (st = check_heads(H, D, "D"))) return st;
  return LI_OK;
}

li_status li_index_decode(const void* q, li_dtype q_dt, const float* w, const void* k_cache,
                          li_dtype k_dt, const float* k_scale, const int64_t* kv_off, int32_t B,
                          int64_t n_tok, int32_t max_len, int32_t H, int32_t D, int32_t k,
                          int32_t* out_idx, float* out_scores, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err.clear();
  li_status st;
  if ((st = check_decode_args(q, q_dt, w, k_cache, k_dt, kv_off, B, n_tok, max_len, H, D, k, out_idx))) return st;
  if ((st = check_ws(ws, ws_bytes, decode_ws(B, n_tok, max_len, k, out_scores != nullptr)))) return st;
  if (B == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_offsets(kv_off, B, n_tok, max_len, s);
        li::validate_bf16(q, (int64_t)B * H * D, li::kBadQ, s);
        li::validate_f32(w, (int64_t)B * H, li::kBadW, s);
        if (k_dt == LI_FP8_E4M3) li::validate_fp8(k_cache, n_tok * D, li::kBadKeys, s);
        else li::validate_bf16(k_cache, n_tok * D, li::kBadKeys, s);
        li::validate_scales(k_scale, n_tok, li::kBadKScale, s);
      })))
    return st;
  trace_begin();
  Carver cv(ws);
  const bool bucket = decode_bucket(n_tok, B, max_len, k);
  float* scores = out_scores ? out_scores : (bucket ? nullptr : (float*)cv.take((size_t)n_tok * 4));
  const li::SelWs sel = carve_sel(cv, B, max_len, li::decode_chunk(n_tok, B), k, bucket);
  if ((st = hip_check(li::launch_decode_score((const uint16_t*)q, w, k_cache, k_dt == LI_FP8_E4M3,
                                              k_scale, kv_off, B, n_tok, max_len, H, k, scores, sel,
                                              s),
                      "decode_score launch", s)))
    return st;
  li::TopkRows tr = {};
  tr.scores = scores;
  tr.mode = li::kRowsOffsets;
  tr.rows = B;
  tr.row_stride = 0;
  tr.kv_off = kv_off;
  tr.G = 1;
  tr.k = k;
  tr.out = out_idx;
  if (bucket) return hip_check(li::launch_topk_bucket(tr, sel, max_len, s), "topk launch", s);
  return hip_check(li::launch_topk_segmented(tr, sel, s), "topk launch", s);
}

li_status li_index_decode_noalloc(const void* q, li_dtype q_dt, const float* w, const void* k_cache,
                                  li_dtype k_dt, const float* k_scale, const int64_t* kv_off, int32_t B,
                                  int64_t n_tok, int32_t max_len, int32_t H, int32_t D, int32_t k,
                                  int32_t* out_idx, float* out_scores, void* stream) {
  g_err.clear();
  li_status st;
  if ((st = check_decode_args(q, q_dt, w, k_cache, k_dt, kv_off, B, n_tok, max_len, H, D, k, out_idx))) return st;
  const size_t need = decode_ws(B, n_tok, max_len, k, out_scores != nullptr);
  if (need > kScratchBytes)
    return fail(LI_E_UNSUPPORTED,
                "li_index_decode_noalloc: this call needs %zu bytes of scratch; the library's static scratch "
                "holds %zu (use li_index_decode with a workspace)", need, kScratchBytes);
  if (B == 0) return LI_OK;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws))) return st;
  return li_index_decode(q, q_dt, w, k_cache, k_dt, k_scale, kv_off, B, n_tok, max_len, H, D, k, out_idx,
                         out_scores, ws, kScratchBytes, stream);
}

size_t li_index_prefill_ws(int32_t T, int32_t L, int32_t k, int32_t has_out_scores) {
  (void)k;
  return prefill_ws(T, L, has_out_scores != 0);
}

li_status li_index_prefill(const void* q, li_dtype q_dt, const float* q_scale, const float* w,
                           const void* k_cache, li_dtype k_dt, const float* k_scale, int32_t T,
                           int32_t L, int32_t qpos0, int32_t H, int32_t D, int32_t k,
                           int32_t* out_idx, float* out_scores, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err.clear();
  if (!q || !w || !k_cache || !out_idx)
    return fail(LI_E_NULL, "q, w, k_cache and out_idx are required");
  if (q_dt != LI_FP8_E4M3 || k_dt != LI_FP8_E4M3)
    return fail(LI_E_DTYPE, "prefill q and k_cache must be LI_FP8_E4M3");
  if (T < 0 || L < 0 || qpos0 < 0 || (int64_t)qpos0 + T > L)
    return fail(LI_E_SHAPE, "need T >= 0, qpos0 >= 0 and qpos0 + T <= L (T=%d L=%d qpos0=%d)", T, L,
                qpos0);
  li_status st;
  if (L > li::kPrefillMaxL)
    return fail(LI_E_SHAPE, "prefill needs L <= %d (got %d)", li::kPrefillMaxL, L);
  if ((st = check_k(k)) || (st = check_heads(H, D, "D"))) return st;
  if (H < kPrefillMinHeads)
    return fail(LI_E_UNSUPPORTED, "prefill needs H >= %d (got %d): the fp8 product's error with fewer heads "
                "can exceed the score tolerance", kPrefillMinHeads, H);
  if ((st = check_ws(ws, ws_bytes, prefill_ws(T, L, out_scores != nullptr)))) return st;
  if (T == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_fp8(q, (int64_t)T * H * D, li::kBadQ, s);
        li::validate_scales(q_scale, T, li::kBadQScale, s);
        li::validate_f32(w, (int64_t)T * H, li::kBadW, s);
        li::validate_fp8(k_cache, (int64_t)L * D, li::kBadKeys, s);
        li::validate_scales(k_scale, L, li::kBadKScale, s);
      })))
    return st;
  trace_begin();
  Carver cv(ws);
  uint2* clist = (uint2*)cv.take((size_t)T * (size_t)L * 8);
  uint32_t* ccnt = (uint32_t*)cv.take((size_t)T * 4);
  uint8_t* uq = (uint8_t*)cv.take((size_t)T * li::kLinRows * 128);
  float* usc = (float*)cv.take((size_t)T * li::kLinRows * 4);
  const li::SelWs sel = carve_sel(cv, T, 0, 0, k, false);
  if ((st = hip_check(li::launch_prefill_linear((const uint8_t*)q, w, T, H, uq, usc, s),
                      "prefill_linear launch", s)))
    return st;
  if ((st = hip_check(li::launch_prefill_score((const uint8_t*)q, q_scale, w, uq, usc,
                                               (const uint8_t*)k_cache, k_scale, T, L, qpos0, H, k,
                                               out_scores, sel, clist, ccnt, s),
                      "prefill_score launch", s)))
    return st;
  li::TopkRows tr = {};
  tr.mode = li::kRowsCausal;
  tr.rows = T;
  tr.row_stride = L;
  tr.n = L;
  tr.qpos0 = qpos0;
  tr.k = k;
  tr.out = out_idx;
  return hip_check(li::launch_topk_list(tr, sel, clist, ccnt, s), "topk launch", s);
}

static li_status check_latent_common(li_dtype q_dt, li_dtype w_dt, li_dtype c_dt, const float* c_scale,
                                     int32_t H, int32_t Dh, int32_t Dc, uint32_t flags) {
  if (q_dt != LI_BF16 || w_dt != LI_BF16 || (c_dt != LI_BF16 && c_dt != LI_FP8_E4M3))
    return fail(LI_E_DTYPE, "q and w_dec must be LI_BF16, the latent LI_BF16 or LI_FP8_E4M3");
  if (c_dt == LI_FP8_E4M3 && !c_scale)
    return fail(LI_E_NULL, "an LI_FP8_E4M3 latent needs its block scales (c_scale [n_tok][Dc/128])");
  if (c_dt == LI_FP8_E4M3 && flags == LI_LATENT_SPLIT_BF16)
    return fail(LI_E_UNSUPPORTED, "LI_LATENT_SPLIT_BF16 takes a bf16 latent only");
  li_status st;
  if ((st = check_heads(H, Dh, "Dh"))) return st;
  if (!dc_ok(Dc)) return fail(LI_E_UNSUPPORTED, "Dc must be 128, 192 or 256 (got %d)", Dc);
  if (flags != LI_LATENT_FP16 && flags != LI_LATENT_SPLIT_BF16)
    return fail(LI_E_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (H < kLatentMinHeads)
    return fail(LI_E_UNSUPPORTED, "the latent forms need H >= %d (got %d): with one head the absorbed "
                "query's rounding can exceed the score tolerance", kLatentMinHeads, H);
  if (c_dt == LI_FP8_E4M3 && H < kLatentFp16MinHeads)
    return fail(LI_E_UNSUPPORTED, "an LI_FP8_E4M3 latent needs H >= %d (got %d)", kLatentFp16MinHeads, H);
  return LI_OK;
}

// The product form a call runs: the split form when asked for, and for a bf16
// latent with fewer heads than the fp16 form is accurate for.
static bool latent_split(uint32_t flags, li_dtype c_dt, int32_t H) {
  return flags == LI_LATENT_SPLIT_BF16 || (c_dt == LI_BF16 && H < kLatentFp16MinHeads);
}

size_t li_latent_score_group_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t G, int32_t H,
                                int32_t Dc, int32_t k, int32_t has_out_scores) {
  (void)k;
  return latent_ws(B, n_tok, max_len, G, H, Dc, has_out_scores != 0);
}

li_status li_latent_score_group(const void* q, li_dtype q_dt, const float* w, const void* w_dec,
                                li_dtype w_dt, const void* latent, li_dtype c_dt,
                                const float* c_scale, const int64_t* kv_off, int32_t B,
                                int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dh,
                                int32_t Dc, int32_t k, int32_t* out_idx, float* out_scores,
                                uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!q || !w || !w_dec || !latent || !kv_off || !out_idx)
    return fail(LI_E_NULL, "q, w, w_dec, latent, kv_off and out_idx are required");
  li_status st;
  if ((st = check_latent_common(q_dt, w_dt, c_dt, c_scale, H, Dh, Dc, flags))) return st;
  if (B < 0 || n_tok < 0 || max_len < 0 || G <= 0)
    return fail(LI_E_SHAPE, "need B, n_tok, max_len >= 0 and G >= 1");
  if ((int64_t)G * n_tok >= (int64_t)1 << 40) return fail(LI_E_UNSUPPORTED, "G * n_tok too large");
  if ((st = check_k(k))) return st;
  if ((st = check_ws(ws, ws_bytes, latent_ws(B, n_tok, max_len, G, H, Dc, out_scores != nullptr))))
    return st;
  if (B == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_offsets(kv_off, B, n_tok, max_len, s);
        li::validate_bf16(q, (int64_t)B * G * H * Dh, li::kBadQ, s);
        li::validate_f32(w, (int64_t)B * G * H, li::kBadW, s);
        li::validate_bf16(w_dec, (int64_t)G * Dc * H * Dh, li::kBadWDec, s);
        li::validate_latent(latent, c_dt == LI_FP8_E4M3, n_tok, Dc, c_scale, !latent_split(flags, c_dt, H), s);
      })))
    return st;
  trace_begin();
  Carver cv(ws);
  uint16_t* qt16 = (uint16_t*)cv.take((size_t)B * G * H * Dc * 4);
  const bool split = latent_split(flags, c_dt, H);
  float* wsc = (float*)cv.take((size_t)B * G * H * 4);
  float* scores = out_scores ? out_scores : (float*)cv.take((size_t)G * (size_t)n_tok * 4);
  const li::SelWs sel = carve_sel(cv, (int64_t)B * G, max_len, li::latent_chunk(n_tok), k, false);
  if ((st = hip_check(li::launch_latent_absorb((const uint16_t*)q, w, (const uint16_t*)w_dec, B, G,
                                               H, Dh, Dc, split, qt16, wsc, s),
                      "latent_absorb launch", s)))
    return st;
  if ((st = hip_check(li::launch_latent_score(qt16, wsc, (const uint16_t*)latent, c_scale, kv_off, B,
                                              n_tok, max_len, G, H, Dc, k, split, c_dt == LI_FP8_E4M3, scores,
                                              sel, s),
                      "latent_score launch", s)))
    return st;
  li::TopkRows tr = {};
  tr.scores = scores;
  tr.mode = li::kRowsOffsets;
  tr.rows = B * G;
  tr.row_stride = n_tok;
  tr.kv_off = kv_off;
  tr.G = G;
  tr.k = k;
  tr.out = out_idx;
  return hip_check(li::launch_topk_segmented(tr, sel, s), "topk launch", s);
}

size_t li_hs_refine_ws(int32_t B, int32_t C, int32_t Gf, int32_t H, int32_t Dc, int32_t k,
                       int32_t has_out_scores) {
  (void)k;
  return hs_ws(B, C, Gf, H, Dc, has_out_scores != 0);
}

li_status li_hs_refine(const int32_t* cand_idx, int32_t C, const void* q, li_dtype q_dt,
                       const float* w, const void* w_dec, li_dtype w_dt, const void* latent,
                       li_dtype c_dt, const float* c_scale, const int64_t* kv_off, int32_t B,
                       int32_t Gf, int32_t H, int32_t Dh, int32_t Dc, int32_t k, int32_t* out_idx,
                       float* out_scores, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream) {
  g_err.clear();
  if (!cand_idx || !q || !w || !w_dec || !latent || !kv_off || !out_idx)
    return fail(LI_E_NULL, "cand_idx, q, w, w_dec, latent, kv_off and out_idx are required");
  li_status st;
  if ((st = check_latent_common(q_dt, w_dt, c_dt, c_scale, H, Dh, Dc, flags))) return st;
  if (B < 0 || Gf <= 0 || C <= 0) return fail(LI_E_SHAPE, "need B >= 0, Gf >= 1 and C >= 1");
  if (C > 65536) return fail(LI_E_UNSUPPORTED, "C must be <= 65536 (got %d)", C);
  if ((st = check_k(k))) return st;
  if ((st = check_ws(ws, ws_bytes, hs_ws(B, C, Gf, H, Dc, out_scores != nullptr)))) return st;
  if (B == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  // The latent cache's length is not an argument here: its rows are checked
  // through the candidates (each inside its request) and kv_off's order.
  // The latent rows are read through the candidates, so they are checked in a
  // second pass, once offsets and candidates are known to be in range.
  if (validate_on() && ((st = run_validation(s, [&] {
                           li::validate_offsets(kv_off, B, INT64_MAX, INT32_MAX, s);
                           li::validate_cands(cand_idx, B, C, kv_off, s);
                           li::validate_bf16(q, (int64_t)B * Gf * H * Dh, li::kBadQ, s);
                           li::validate_f32(w, (int64_t)B * Gf * H, li::kBadW, s);
                           li::validate_bf16(w_dec, (int64_t)Gf * Dc * H * Dh, li::kBadWDec, s);
                         })) ||
                        (st = run_validation(s, [&] {
                           li::validate_cand_latent(cand_idx, B, C, kv_off, latent, c_dt == LI_FP8_E4M3, Dc, c_scale,
                                                    !latent_split(flags, c_dt, H), s);
                         }))))
    return st;
  trace_begin();
  Carver cv(ws);
  uint16_t* qt16 = (uint16_t*)cv.take((size_t)B * Gf * H * Dc * 4);
  const bool split = latent_split(flags, c_dt, H);
  float* wsc = (float*)cv.take((size_t)B * Gf * H * 4);
  float* scores = out_scores ? out_scores : (float*)cv.take((size_t)B * Gf * (size_t)C * 4);
  if ((st = hip_check(li::launch_latent_absorb((const uint16_t*)q, w, (const uint16_t*)w_dec, B, Gf,
                                               H, Dh, Dc, split, qt16, wsc, s),
                      "latent_absorb launch", s)))
    return st;
  if ((st = hip_check(li::launch_hs_score(qt16, wsc, (const uint16_t*)latent, c_scale, kv_off,
                                          cand_idx, C, B, Gf, H, Dc, split, c_dt == LI_FP8_E4M3, scores, s),
                      "hs_score launch", s)))
    return st;
  li::TopkRows tr = {};
  tr.scores = scores;
  tr.mode = li::kRowsCands;
  tr.rows = B * Gf;
  tr.cand = cand_idx;
  tr.C = C;
  tr.G = Gf;
  tr.k = k;
  tr.out = out_idx;
  return hip_check(li::launch_topk(tr, s), "topk launch", s);
}

size_t li_latent_append_ws(int32_t M, int32_t d_model, int32_t Dc, li_dtype c_dt) {
  if (M <= 0 || d_model < 64 || d_model % 64 != 0 || !dc_ok(Dc)) return 0;
  const int32_t S = li::append_splits(M, d_model);
  return S > 1 || c_dt == LI_FP8_E4M3 ? align_up((size_t)S * M * Dc * 4) : 0;
}

li_status li_latent_append(const void* h, li_dtype h_dt, const void* w_enc, li_dtype w_dt,
                           const int64_t* dst_row, int32_t M, int32_t d_model, int32_t Dc, void* latent,
                           li_dtype c_dt, float* c_scale, int64_t n_tok, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!w_enc || !latent) return fail(LI_E_NULL, "w_enc and latent are required");
  if (M > 0 && (!h || !dst_row)) return fail(LI_E_NULL, "h and dst_row are required when M > 0");
  if (h_dt != LI_BF16 || w_dt != LI_BF16) return fail(LI_E_DTYPE, "h and w_enc must be LI_BF16");
  if (c_dt != LI_BF16 && c_dt != LI_FP8_E4M3) return fail(LI_E_DTYPE, "the latent must be LI_BF16 or LI_FP8_E4M3");
  if (c_dt == LI_FP8_E4M3 && !c_scale) return fail(LI_E_NULL, "an LI_FP8_E4M3 latent needs c_scale [n_tok][Dc/128]");
  if (M < 0 || d_model <= 0 || n_tok <= 0) return fail(LI_E_SHAPE, "need M >= 0, d_model >= 1 and n_tok >= 1");
  if (d_model % 64 != 0) return fail(LI_E_UNSUPPORTED, "d_model must be a multiple of 64 (got %d)", d_model);
  if (!dc_ok(Dc)) return fail(LI_E_UNSUPPORTED, "Dc must be 128, 192 or 256 (got %d)", Dc);
  li_status st;
  if ((st = check_ws(ws, ws_bytes, li_latent_append_ws(M, d_model, Dc, c_dt)))) return st;
  if (M == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_dst_rows(dst_row, M, n_tok, s);
        li::validate_bf16(h, (int64_t)M * d_model, li::kBadHidden, s);
        li::validate_bf16(w_enc, (int64_t)Dc * d_model, li::kBadWEnc, s);
      })))
    return st;
  trace_begin();
  return hip_check(li::launch_latent_append((const uint16_t*)h, (const uint16_t*)w_enc, dst_row, M, d_model, Dc,
                                            (float*)ws, (uint16_t*)latent, c_dt == LI_FP8_E4M3, c_scale, s),
                   "latent_append launch", s);
}

size_t li_sparse_attention_ws(int32_t B, int32_t H, int32_t k) {
  if (B <= 0 || H <= 0 || H % 64 != 0 || k <= 0) return 0;
  const size_t rows = (size_t)li::attention_splits(B, H, k) * B * H;
  return align_up(rows * 512 * 4) + align_up(rows * 2 * 4);
}

li_status li_sparse_attention(const void* q, li_dtype q_dt, const void* kv, li_dtype kv_dt, const int32_t* idx,
                              const int64_t* kv_off, int32_t B, int64_t n_tok, int32_t H, int32_t Dk, int32_t Dv,
                              int32_t k, float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!q || !kv || !idx || !kv_off || !out) return fail(LI_E_NULL, "q, kv, idx, kv_off and out are required");
  if (q_dt != LI_BF16 || kv_dt != LI_BF16) return fail(LI_E_DTYPE, "q and kv must be LI_BF16");
  if (B < 0 || n_tok <= 0 || H <= 0 || k <= 0) return fail(LI_E_SHAPE, "need B >= 0, n_tok >= 1, H >= 1 and k >= 1");
  if (Dk != 576 || Dv != 512) return fail(LI_E_UNSUPPORTED, "Dk must be 576 and Dv 512 (got %d, %d)", Dk, Dv);
  if (H % 64 != 0 || H > 256) return fail(LI_E_UNSUPPORTED, "H must be 64, 128, 192 or 256 (got %d)", H);
  if (k > 65536) return fail(LI_E_UNSUPPORTED, "k must be <= 65536 (got %d)", k);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return fail(LI_E_SHAPE, "scale must be finite");
  li_status st;
  if ((st = check_ws(ws, ws_bytes, li_sparse_attention_ws(B, H, k)))) return st;
  if (B == 0) return LI_OK;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_offsets(kv_off, B, n_tok, INT32_MAX, s);
        li::validate_cands(idx, B, k, kv_off, s);
        li::validate_bf16(q, (int64_t)B * H * Dk, li::kBadQ, s);
        li::validate_bf16(kv, n_tok * Dk, li::kBadKeys, s);
      })))
    return st;
  trace_begin();
  Carver cv(ws);
  const size_t rows = (size_t)li::attention_splits(B, H, k) * B * H;
  float* o_part = (float*)cv.take(rows * 512 * 4);
  float* ml_part = (float*)cv.take(rows * 2 * 4);
  return hip_check(li::launch_sparse_attention((const uint16_t*)q, (const uint16_t*)kv, idx, kv_off, B, H, k, scale,
                                               o_part, ml_part, out, s),
                   "sparse_attention launch", s);
}

size_t li_key_row_bytes(int32_t D, li_dtype dt) {
  if (D <= 0) return 0;
  if (dt == LI_FP8_E4M3) return (size_t)D + 4;
  if (dt == LI_BF16) return (size_t)D * 2;
  return 0;
}

size_t li_latent_row_bytes(int32_t Dc, li_dtype dt) {
  if (Dc <= 0) return 0;
  if (dt == LI_FP8_E4M3) return (size_t)Dc + 4 * (size_t)((Dc + 127) / 128);
  if (dt == LI_BF16) return (size_t)Dc * 2;
  return 0;
}

int32_t li_indexcache_plan(const uint8_t* roles, int32_t n_layers, int32_t retain_every, int32_t* src) {
  g_err.clear();
  if (!src) return -fail(LI_E_NULL, "src is required");
  if (n_layers < 1) return -fail(LI_E_SHAPE, "n_layers must be >= 1 (got %d)", n_layers);
  if (!roles && retain_every < 1) return -fail(LI_E_SHAPE, "retain_every must be >= 1 (got %d)", retain_every);
  if (roles && roles[0] != 1) return -fail(LI_E_SHAPE, "the first layer must be F (roles[0] = 1)");
  int32_t full = 0, last = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const bool f = roles ? roles[l] != 0 : l % retain_every == 0;
    if (f) {
      last = l;
      ++full;
    }
    src[l] = last;
  }
  return full;
}

size_t li_topk_ws(int32_t rows, int32_t n, int32_t k) {
  (void)rows;
  (void)n;
  (void)k;
  return 0;
}

li_status li_topk(const float* scores, int64_t row_stride, const int32_t* row_len, int32_t rows,
                  int32_t n, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!scores || !out_idx) return fail(LI_E_NULL, "scores and out_idx are required");
  if (rows < 0 || n < 0 || row_stride < n)
    return fail(LI_E_SHAPE, "need rows >= 0 and 0 <= n <= row_stride");
  li_status st;
  if ((st = check_k(k))) return st;
  if ((st = check_ws(ws, ws_bytes, li_topk_ws(rows, n, k)))) return st;
  if (rows == 0) return LI_OK;
  li::TopkRows tr = {};
  tr.scores = scores;
  tr.mode = li::kRowsDense;
  tr.rows = rows;
  tr.row_stride = row_stride;
  tr.row_len = row_len;
  tr.n = n;
  tr.k = k;
  tr.out = out_idx;
  hipStream_t s = (hipStream_t)stream;
  if (validate_on() && (st = run_validation(s, [&] {
        li::validate_row_len(row_len, rows, row_stride, s);
        li::validate_score_rows(scores, row_stride, rows, n, row_len, s);
      })))
    return st;
  trace_begin();
  return hip_check(li::launch_topk(tr, s), "topk launch", s);
}

}  // extern "C"
