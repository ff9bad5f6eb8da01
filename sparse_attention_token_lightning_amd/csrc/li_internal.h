// Host-side launchers shared between the kernel files and the C-ABI layer.
// Every launcher only enqueues work on `stream` and returns the launch status.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "li_select.h"

namespace li {

// Measurement hook (li_trace_events): the (start, stop) events to attach to
// the next kernel launch of the current entry point, or two nulls.
void trace_next(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the entry points is launched through here.  With the
// measurement hook on, the launch carries a (start, stop) event pair that
// the runtime sets to the kernel's own start and end, so no event marker
// sits between two kernels of a call.
template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  trace_next(&start, &stop);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, start, stop, 0u, args...);
  return hipGetLastError();
}

// How the top-k kernel finds row r of the score matrix.
enum TopkMode : int32_t {
  kRowsDense = 0,    // row r at scores + r*row_stride, length row_len[r] or n
  kRowsOffsets = 1,  // row r = b*G + l at scores + l*plane + kv_off[b], length kv_off[b+1]-kv_off[b]
  kRowsCausal = 2,   // row t at scores + t*row_stride, length min(n, qpos0 + t + 1)
  kRowsCands = 3,    // row r = b*G + f at scores + r*C, length = valid candidates of b,
                     // positions mapped through cand[b][.]
};

struct TopkRows {
  const float* scores;
  int32_t mode;
  int32_t rows;
  int64_t row_stride;      // dense / causal: row stride; offsets: plane stride (n_tok)
  const int32_t* row_len;  // dense, may be null
  int32_t n;               // dense: default length; causal: L
  const int64_t* kv_off;   // offsets
  int32_t G;               // offsets / candidates: rows per request
  int32_t qpos0;           // causal
  const int32_t* cand;     // candidates [B][C]
  int32_t C;
  int32_t k;
  int32_t* out;            // [rows][k]
};

// Top-k with the level-0 histogram built on the fly (one workgroup per row).
hipError_t launch_topk(const TopkRows& a, hipStream_t stream);
// Top-k from the scan's partial histograms: many workgroups per row collect
// candidates; the last one of each row finishes it (one launch).
hipError_t launch_topk_segmented(const TopkRows& a, const SelWs& ws, hipStream_t stream);
// LDS candidate capacity of the segmented top-k's final step for a given k.
int32_t seg_cap_for(int32_t k);
// Scores per collect segment of the segmented top-k for `rows` rows of up to
// max_len scores (larger segments when the grid would not fit the GPU at once).
int64_t seg_len_for(int64_t rows, int64_t max_len);
// Bucket mode (SelWs::bucket, decode): one workgroup per row reads the scan's
// prefix partials and bin-ordered candidate lists.  Used when a row spans at
// most kBucketMaxNwg scan workgroups, each of at least 2k positions or at most
// 4096 (every key then fits the scan's LDS staging), max_len <= kBucketMaxLen
// (the LDS position bitmaps) and the LDS left for the threshold bin's keys is
// useful.
constexpr int kBucketMaxNwg = 32;
constexpr int64_t kBucketMaxLen = 1 << 17;  // also keeps the packed word prefixes exact
constexpr int64_t kBucketLds = 147456;  // dynamic LDS of the bucket top-k kernel
constexpr int32_t kBucketStageK = 4096;  // output rows up to this k are staged in LDS
int32_t bucket_cap_for(int32_t k, int64_t max_len);
bool bucket_ok(int64_t nwg, int64_t chunk, int32_t k, int64_t max_len);
hipError_t launch_topk_bucket(const TopkRows& a, const SelWs& ws, int64_t max_len, hipStream_t stream);
// Top-k from scan-built thresholds, one workgroup per row collecting its own candidates.
hipError_t launch_topk_self(const TopkRows& a, const SelWs& ws, hipStream_t stream);
// Top-k of causal rows (a.n = L, a.qpos0, a.row_stride = L) given as the
// prefill scan's candidate lists (list [rows][L] pairs, lcnt [rows]).
hipError_t launch_topk_list(const TopkRows& a, const SelWs& ws, const uint2* list, const uint32_t* lcnt,
                            hipStream_t stream);
// Positions of one row covered by one scan workgroup (decode / latent).
int64_t decode_chunk(int64_t n_tok, int32_t B);
// Longest fp8 request of the decode scan: its keys are addressed with 32-bit
// byte offsets (position * 128 plus at most 4095 within a tile).
constexpr int32_t kDecodeFp8MaxLen = (1 << 25) - 4096;
int64_t latent_chunk(int64_t n_tok);

// Decode scan: scores[kv_off[b] + s] for every request b and s < L_b; rows
// longer than k also get their partial level-0 histograms in `sel`.
hipError_t launch_decode_score(const uint16_t* q, const float* w, const void* kc, bool kc_fp8,
                               const float* k_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t H, int32_t k,
                               float* scores, const SelWs& sel, hipStream_t stream);

// Prefill: u = sum_h w_h q_hat_h per token as kLinRows fp8 rows + scales
// (uq [T][4][128] bytes, usc [T][4]), then the causal scan, which appends
// each row's candidates (keys that can still be among its top k) to a list
// and leaves the threshold bin of rows with more than k visible keys in
// sel.thr.  kPrefillMaxL bounds the cache length so that the candidate rows
// of one wave fit one buffer resource.
constexpr int kLinRows = 4;
constexpr int32_t kPrefillMaxL = 1 << 26;
hipError_t launch_prefill_linear(const uint8_t* q, const float* w, int32_t T, int32_t H, uint8_t* uq,
                                 float* usc, hipStream_t stream);
// scores: the dense [T][L] output (out_scores) or null; clist [T][L] (key,
// position) pairs and ccnt [T] receive each row's candidate list.
hipError_t launch_prefill_score(const uint8_t* q, const float* q_scale, const float* w,
                                const uint8_t* uq, const float* usc, const uint8_t* kc,
                                const float* k_scale, int32_t T, int32_t L, int32_t qpos0, int32_t H,
                                int32_t k, float* scores, const SelWs& sel, uint2* clist, uint32_t* ccnt,
                                hipStream_t stream);

// Latent absorption: qt16[b][l][h][Dc] (range-scaled by 2^e per row) and
// wsc[b][l][h] = w * 2^-e.  The row is fp16, or with split two bf16 parts,
// hi at qt16[row] and lo at qt16[B*G*H + row] (qt16 then holds 2*B*G*H*Dc).
hipError_t launch_latent_absorb(const uint16_t* q, const float* w, const uint16_t* w_dec,
                                int32_t B, int32_t G, int32_t H, int32_t Dh, int32_t Dc, bool split,
                                uint16_t* qt16, float* wsc, hipStream_t stream);

// Latent scan over contiguous ragged rows: scores[l*n_tok + kv_off[b] + s];
// rows (b, l) longer than k also get their partial histograms in `sel`.
hipError_t launch_latent_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                               const float* c_scale, const int64_t* kv_off, int32_t B,
                               int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dc,
                               int32_t k, bool split, bool fp8, float* scores, const SelWs& sel,
                               hipStream_t stream);

// HS gather scan: scores[(b*Gf + f)*C + j] for the valid candidates j of b.
hipError_t launch_hs_score(const uint16_t* qt16, const float* wsc, const uint16_t* latent,
                           const float* c_scale, const int64_t* kv_off, const int32_t* cand,
                           int32_t C, int32_t B, int32_t Gf, int32_t H, int32_t Dc, bool split, bool fp8,
                           float* scores, hipStream_t stream);

// Latent-cache append: latent[dst[m]] = bf16(sum_i h[m][i] * w_enc[c][i]).
// K is split over append_splits(M, d_model) workgroups; with more than one
// split (and always for fp8 output), `part` ([S][M][Dc] fp32) holds the partial sums.
int32_t append_splits(int32_t M, int32_t d_model);

// Sparse attention over selected rows (Dk = 576, Dv = 512, H a multiple of
// 64): token splits write partial outputs o_part [S][B][H][512] and (max, sum)
// pairs ml_part [S][B][H][2]; a second kernel combines them into out.
int32_t attention_splits(int32_t B, int32_t H, int32_t K);
hipError_t launch_sparse_attention(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int64_t* kv_off,
                                   int32_t B, int32_t H, int32_t K, float scale, float* o_part, float* ml_part,
                                   float* out, hipStream_t stream);
hipError_t launch_latent_append(const uint16_t* h, const uint16_t* w_enc, const int64_t* dst, int32_t M,
                                int32_t d_model, int32_t Dc, float* part, uint16_t* latent, bool fp8, float* c_scale,
                                hipStream_t stream);

// Read-bandwidth probe (measurement aid): streams bytes / 16 16-byte words of
// p (16-byte aligned) and writes one fold per wave into sink
// (LI_READ_PROBE_SINK_WORDS words).
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* sink, hipStream_t stream);
// Matrix-core rate probe (measurement aid): form LI_MFMA_PROBE_*, operands
// constant or random, iters iterations of LI_MFMA_PROBE_PRODUCTS_PER_ITER
// products per wave; sink LI_MFMA_PROBE_SINK_WORDS floats, clk
// LI_MFMA_PROBE_CLOCK_WORDS words.
hipError_t launch_mfma_probe(int form, bool random_operands, int iters, float* sink, uint32_t* clk,
                             hipStream_t stream);

// Opt-in input checks (LI_DEBUG_VALIDATE): validate_begin clears the device
// record, the validate_* calls enqueue one check each, validate_end waits for
// them and returns the first failed check (0 = none) and its element index.
enum ValidateCheck : uint32_t {
  kBadOffsetRange = 1,
  kBadOffsetOrder,
  kBadLength,
  kBadKScale,
  kBadQScale,
  kBadCScale,
  kBadW,
  kBadQ,
  kBadKeys,
  kBadLatent,
  kBadWDec,
  kBadCandidate,
  kBadCandidateOrder,
  kBadScores,
  kBadRowLen,
  kBadDstRow,
  kBadHidden,
  kBadWEnc,
  kBadLatentRange,
  kBadCScaleRange,
};
hipError_t validate_begin(hipStream_t s);
void validate_offsets(const int64_t* off, int32_t B, int64_t n_tok, int32_t max_len, hipStream_t s);
void validate_scales(const float* p, int64_t n, uint32_t check, hipStream_t s);
void validate_f32(const float* p, int64_t n, uint32_t check, hipStream_t s);
void validate_bf16(const void* p, int64_t n, uint32_t check, hipStream_t s);
void validate_fp8(const void* p, int64_t n, uint32_t check, hipStream_t s);
void validate_cands(const int32_t* cand, int32_t B, int32_t C, const int64_t* off, hipStream_t s);
// Latent codes and scales (ceil(Dc / 128) block scales per row for fp8, one
// optional row scale for bf16); with fp16_form also the fp16-range limits.
void validate_latent(const void* latent, bool fp8, int64_t n_tok, int32_t Dc, const float* c_scale,
                     bool fp16_form, hipStream_t s);
// The same over the rows kv_off[b] + cand[b][j] of valid candidates only.
void validate_cand_latent(const int32_t* cand, int32_t B, int32_t C, const int64_t* off, const void* latent,
                          bool fp8, int32_t Dc, const float* c_scale, bool fp16_form, hipStream_t s);
void validate_score_rows(const float* p, int64_t stride, int32_t rows, int32_t n, const int32_t* len,
                         hipStream_t s);
void validate_row_len(const int32_t* len, int32_t rows, int64_t stride, hipStream_t s);
void validate_dst_rows(const int64_t* dst, int32_t M, int64_t n_tok, hipStream_t s);
hipError_t validate_end(hipStream_t s, uint32_t* check, int64_t* index);
const char* validate_name(uint32_t check);

}  // namespace li
