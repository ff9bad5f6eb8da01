/*
 * li.h — C ABI of the MI355X (gfx950) lightning-indexer library.
 *
 * The operation (sources are page titles and sections):
 *   For each query token the lightning indexer gives every cached position the
 *   query may attend a score, and the k best-scoring positions (k = 2,048 in
 *   the pages) form the index tensor that sparse attention reads.  ("IndexCache: Cross-Layer Index Reuse for Sparse
 *   Attention", Symbol Map and Deep Dive; "Multi-layer Indexer: Overlapping
 *   Selection and Attention in DeepSeek Sparse Attention", The abstract.)
 *   The score this library computes is
 *       S[s] = sum_h w[h] * ReLU(q[h] . k[s])
 *   with per-token scales applied to the dequantised operands, and ties in the
 *   selection go to the lower position.
 *   LatentIndex variant: a group of layers shares one latent cache; each layer's
 *   key decoder is folded into its query, so the shared cache is scored as
 *   stored and every layer still selects on its own.  HS variant: the anchor
 *   layer's selection is the pool from which the follower layers pick.  ("LatentIndex:
 *   Cross-Layer Sharing with Layer-Specific Selection for Sparse Attention",
 *   Abstract and Figure 1.)  Shapes: 64 indexer heads x 128 dims per key
 *   (same page, Table 5).
 *
 * Conventions for every entry point:
 *   - Every array pointer is caller-owned DEVICE memory (e.g. a torch tensor's
 *     data_ptr()); nothing is copied to or from the host.  The library keeps no
 *     state between calls and never allocates device memory: scratch space is
 *     the caller's workspace `ws` of `ws_bytes` bytes, sized by the matching
 *     li_*_ws() query (it may be NULL when that query returns 0).  The query's
 *     has_out_scores flag says whether the call will be given an out_scores
 *     buffer; without one the scores live in the workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue kernels on it and return without synchronising; results are
 *     ready when the stream has drained.  Ragged lengths are read on the
 *     device from `kv_off`, so the host never reads device memory.  A call
 *     may be captured into a HIP graph (stream capture) and replayed; the
 *     workspace and outputs it was given are then reused by every replay.
 *   - Errors found on the host (a NULL required pointer, a bad size, an
 *     unsupported dtype or shape, a workspace that is too small) return a
 *     status before anything is enqueued.  A failed kernel launch returns
 *     LI_E_HIP; li_last_error() then holds the HIP error text (thread-local).
 *   - Device contents are not validated: kv_off must be non-decreasing with
 *     kv_off[0] >= 0, lengths must not exceed max_len, scales must be finite
 *     and positive, inputs must not hold NaN/Inf codes, candidate rows must be
 *     ascending inside [0, L_b) with -1 only at their end.  Otherwise the
 *     results are undefined, and an offset or candidate pointing past its
 *     buffer makes the kernels read past it too.
 *   - Debug validation: with the environment variable LI_DEBUG_VALIDATE set
 *     (to anything but "" or "0") at the time of a call, the entry point
 *     first runs device-side checks of those preconditions on its
 *     inputs, waits for them on `stream` (so such calls synchronise and must
 *     not be captured into a graph) and returns LI_E_VALUE if one fails;
 *     li_last_error() names the failed check and the element index.
 *   - Output index rows hold the kept positions in ascending order; a row
 *     with fewer than k visible positions returns all of them and pads the
 *     rest of its k slots with -1.  Scores compare as IEEE values with
 *     -0 == +0; the lower position wins a tie.
 *   - Element types: LI_BF16 (bfloat16), LI_FP8_E4M3 (OCP FP8 E4M3FN: bias 7,
 *     max 448, no infinities), LI_FP16 (IEEE binary16), LI_FP32.
 */
#ifndef LI_H
#define LI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t li_status;
#define LI_OK 0
#define LI_E_NULL 1        /* a required pointer is NULL */
#define LI_E_SHAPE 2       /* a size is negative, zero where it must not be, or inconsistent */
#define LI_E_DTYPE 3       /* an element type this entry point does not take */
#define LI_E_WORKSPACE 4   /* ws_bytes is smaller than the li_*_ws() query */
#define LI_E_UNSUPPORTED 5 /* a shape outside the supported set (see each entry point) */
#define LI_E_HIP 6         /* a HIP runtime call or kernel launch failed */
#define LI_E_VALUE 7       /* LI_DEBUG_VALIDATE only: a device input broke a precondition */

typedef int32_t li_dtype;
#define LI_BF16 0
#define LI_FP8_E4M3 1
#define LI_FP16 2
#define LI_FP32 3

/* Largest k any entry point takes. */
#define LI_MAX_K 16384

/* ---------------------------------------------------------------------------
 * li_index_decode — one decode step of the DSA lightning indexer.
 *
 * B requests with one query token each score their own ragged slice of a
 * shared key cache and keep their top-k.  Request b owns cache rows
 * [kv_off[b], kv_off[b+1]); its L_b = kv_off[b+1] - kv_off[b] positions are
 * all visible.  Score of position s of request b (row r = kv_off[b] + s):
 *     S = sum_h w[b][h] * ReLU( (q[b][h] . dec(k_cache[r])) * k_scale[r] )
 *
 *   q        [B][H][D]   LI_BF16
 *   w        [B][H]      fp32 head weights
 *   k_cache  [n_tok][D]  LI_BF16 or LI_FP8_E4M3 (one key per token, shared by all heads)
 *   k_scale  [n_tok]     fp32 per-token dequantisation scale, or NULL (= 1)
 *   kv_off   [B+1]       int64, device
 *   n_tok    rows in k_cache (>= kv_off[B]); max_len >= every L_b (grid sizing);
 *            with LI_FP8_E4M3 keys max_len <= 33550336 (else LI_E_UNSUPPORTED)
 *   H        1..64 heads; D must be 128; 1 <= k <= LI_MAX_K
 *   out_idx  [B][k]      int32 positions in [0, L_b), ascending, -1 padded
 *   out_scores [n_tok]   fp32 score of every cache row, or NULL
 *
 * Selection (both ways give the same indices): when max_len <= 2^17 and a
 * request spans at most 32 scan workgroups of at least 2k positions each (a
 * workgroup covers 512 .. 8192 positions, more as n_tok grows: k = 2048 takes
 * this way from about 2M cached tokens on), every scan workgroup leaves its keys at or
 * above its own k-th largest level-0 bin as (key, position) lists ordered by
 * bin, and one workgroup per request reads only the part at or above the
 * request's threshold bin; the workspace then holds those lists (8 bytes per
 * key) and no score buffer.  Otherwise many workgroups per request collect
 * candidates from a score buffer in the workspace (4 bytes per key, unless
 * out_scores is given) and the last one to finish selects.
 * ------------------------------------------------------------------------- */
li_status li_index_decode(const void* q, li_dtype q_dt, const float* w, const void* k_cache,
                          li_dtype k_dt, const float* k_scale, const int64_t* kv_off, int32_t B,
                          int64_t n_tok, int32_t max_len, int32_t H, int32_t D, int32_t k,
                          int32_t* out_idx, float* out_scores, void* ws, size_t ws_bytes,
                          void* stream);
size_t li_index_decode_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t k,
                          int32_t has_out_scores);

/* ---------------------------------------------------------------------------
 * li_index_decode_noalloc — li_index_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, kernels and results, with the
 * workspace taken from a static device array of LI_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing; the first call on a device looks the array's address up
 * (hipGetSymbolAddress).
 *
 *   A call whose li_index_decode_ws(B, n_tok, max_len, k, out_scores != NULL)
 *   exceeds LI_NOALLOC_SCRATCH_BYTES returns LI_E_UNSUPPORTED before any
 *   device work (the B = 32, 131072-token decode needs about 34 MiB).
 *   Every call on one GPU shares that GPU's array: calls that can overlap on
 *   one GPU (different streams, or concurrent host threads) race and must be
 *   serialised by the caller.  Nothing in the array needs to start at zero:
 *   the kernels write every scratch value they read in the same call.
 * ------------------------------------------------------------------------- */
#define LI_NOALLOC_SCRATCH_BYTES 67108864u /* 64 MiB */
li_status li_index_decode_noalloc(const void* q, li_dtype q_dt, const float* w, const void* k_cache,
                                  li_dtype k_dt, const float* k_scale, const int64_t* kv_off, int32_t B,
                                  int64_t n_tok, int32_t max_len, int32_t H, int32_t D, int32_t k,
                                  int32_t* out_idx, float* out_scores, void* stream);

/* ---------------------------------------------------------------------------
 * li_index_prefill — the indexer over a prefill chunk of one sequence.
 *
 * T new query tokens at positions qpos0 .. qpos0+T-1 of an L-token cache that
 * already holds their keys.  Row t sees positions s <= qpos0 + t (causal,
 * diagonal included).  Score:
 *     S[t][s] = sum_h w[t][h] * ReLU( q_scale[t] * k_scale[s] * (dec(q[t][h]) . dec(k_cache[s])) )
 *
 *   q        [T][H][D]  LI_FP8_E4M3 ; q_scale [T] fp32 or NULL (= 1)
 *   w        [T][H]     fp32
 *   k_cache  [L][D]     LI_FP8_E4M3 ; k_scale [L] fp32 or NULL (= 1)
 *   0 <= qpos0, qpos0 + T <= L <= 2^26;  H 8..64;  D must be 128;  1 <= k <= LI_MAX_K
 *   out_idx    [T][k]   int32 positions, ascending, -1 padded
 *   out_scores [T][L]   fp32 or NULL; masked positions hold -inf
 *
 * The scan keeps, for each row, only the keys that can still be among its
 * top k: those whose level-0 bin is at or above a floor, the bin of the k-th
 * largest key seen so far, which rises as the row's keys go by.  The selection
 * reads these (key, position) lists instead of all T x L scores.  The
 * workspace (li_index_prefill_ws) sizes them for the worst case, 8 bytes per
 * (t, s) pair: about T * L * 8 bytes.
 *
 * The products run on fp8 matrix cores, whose accumulation error is relative
 * to sum_d |q_d k_d| of a head rather than to its dot product; with fewer than
 * 8 heads one cancelling head can exceed the score tolerance
 * (|dS| <= 2e-3 * sum_h |w_h x_h|), so H < 8 returns LI_E_UNSUPPORTED.
 * Measured at H = 8: within 8.3e-5 of that sum on N(0,1) inputs, 4.8e-4 with
 * query elements spread over 2^-9 .. 2^0; at H = 64 within 1.3e-5.
 * ------------------------------------------------------------------------- */
li_status li_index_prefill(const void* q, li_dtype q_dt, const float* q_scale, const float* w,
                           const void* k_cache, li_dtype k_dt, const float* k_scale, int32_t T,
                           int32_t L, int32_t qpos0, int32_t H, int32_t D, int32_t k,
                           int32_t* out_idx, float* out_scores, void* ws, size_t ws_bytes,
                           void* stream);
size_t li_index_prefill_ws(int32_t T, int32_t L, int32_t k, int32_t has_out_scores);

/* Selects the MFMA operand form of the absorbed latent queries.  Both forms
 * need H >= 2 (with one head the absorbed query's rounding can exceed the
 * score tolerance: LI_E_UNSUPPORTED). */
#define LI_LATENT_FP16 0u /* fp16 absorbed query (per-row power-of-two range scaling), latent
                             converted bf16 -> fp16 on the fly; requires latent magnitudes
                             within fp16 range (|c| <= 65504).  One product per element;
                             score error up to about 2e-4 of sum_h |w_h x_h| at H = 64 and
                             4e-4 at H = 16 (measured on N(0,1) latents).  With fewer than
                             16 heads a bf16 latent is scored in the LI_LATENT_SPLIT_BF16
                             form instead (the fp16 form's error nears the tolerance
                             there), and an LI_FP8_E4M3 latent is LI_E_UNSUPPORTED. */
#define LI_LATENT_SPLIT_BF16 1u /* absorbed query as two bf16 parts, hi + lo (lo = the bf16
                                   rounding of the exact residual), against the bf16 latent as
                                   stored (any magnitude bf16 holds).  Two products per element
                                   (about 1.8x the fp16 form's scan time); score error up to
                                   about 2e-6 of sum_h |w_h x_h| (same measurement). */

/* ---------------------------------------------------------------------------
 * li_latent_score_group — LatentIndex: G layers score one shared latent cache.
 *
 * Layer l's key decoder w_dec[l] (stored [Dc][H*Dh]; head h's key is
 * k[j] = sum_c w_dec[l][c][h*Dh + j] * c[c]) is absorbed into the query,
 *     qt[b][l][h][c] = sum_j w_dec[l][c][h*Dh + j] * q[b][l][h][j],
 * and every position s of request b is scored for every layer in one pass
 * over the latent cache:
 *     S_l[s] = sum_h w[b][l][h] * ReLU( c_scale[r] * (qt[b][l][h] . dec(latent[r])) )
 * Each layer then keeps its own top-k (layer-specific selection).
 *
 *   q       [B][G][H][Dh] LI_BF16;  w [B][G][H] fp32
 *   w_dec   [G][Dc][H*Dh] LI_BF16
 *   latent  [n_tok][Dc]   LI_BF16 with c_scale [n_tok] fp32 or NULL (= 1), or
 *           LI_FP8_E4M3 with c_scale [n_tok][ceil(Dc/128)] fp32 (required): one scale
 *           per 128-value block counted from the row's start (Dc = 192: blocks of
 *           128 and 64 values); for the fp16 product each code is taken times
 *           the scale's power of two (exact) and times its mantissa factor
 *           (rounded to fp16), rounding once to fp16 (fp16 form only)
 *   kv_off  [B+1] int64, device;  max_len >= every L_b
 *   G >= 1;  H 2..64 (16..64 for LI_FP8_E4M3);  Dh must be 128;  Dc 128, 192 or 256;
 *   1 <= k <= LI_MAX_K
 *   out_idx    [B][G][k]  int32 positions, ascending, -1 padded
 *   out_scores [G][n_tok] fp32 or NULL
 *   flags      LI_LATENT_FP16 or LI_LATENT_SPLIT_BF16
 * ------------------------------------------------------------------------- */
li_status li_latent_score_group(const void* q, li_dtype q_dt, const float* w, const void* w_dec,
                                li_dtype w_dt, const void* latent, li_dtype c_dt,
                                const float* c_scale, const int64_t* kv_off, int32_t B,
                                int64_t n_tok, int32_t max_len, int32_t G, int32_t H, int32_t Dh,
                                int32_t Dc, int32_t k, int32_t* out_idx, float* out_scores,
                                uint32_t flags, void* ws, size_t ws_bytes, void* stream);
size_t li_latent_score_group_ws(int32_t B, int64_t n_tok, int32_t max_len, int32_t G, int32_t H,
                                int32_t Dc, int32_t k, int32_t has_out_scores);

/* ---------------------------------------------------------------------------
 * li_hs_refine — HS followers rescore only the anchor's candidate set.
 *
 * cand_idx [B][C] holds the anchor's kept positions for each request in
 * ascending order, -1 padded (e.g. out_idx of li_index_decode called with
 * k = C).  Each follower layer f < Gf absorbs its decoder into its query (as in
 * li_latent_score_group), scores the latent rows kv_off[b] + cand_idx[b][j] of
 * the valid candidates, and keeps its own top-k among them.
 *
 *   q [B][Gf][H][Dh] LI_BF16; w [B][Gf][H] fp32; w_dec [Gf][Dc][H*Dh] LI_BF16
 *   latent [n_tok][Dc] LI_BF16 with c_scale [n_tok] or NULL, or LI_FP8_E4M3 with
 *   block scales [n_tok][ceil(Dc/128)] (as in li_latent_score_group); kv_off [B+1] int64
 *   1 <= C <= 65536; Gf >= 1; H 2..64 (16..64 for LI_FP8_E4M3); Dh 128; Dc 128, 192 or 256;
 *   1 <= k <= LI_MAX_K
 *   out_idx    [B][Gf][k] int32 TOKEN positions (taken from cand_idx), ascending, -1 padded
 *   out_scores [B][Gf][C] fp32 score of candidate slot j, or NULL (slots past
 *              the valid candidates are not written)
 *   flags      LI_LATENT_FP16 or LI_LATENT_SPLIT_BF16
 * ------------------------------------------------------------------------- */
li_status li_hs_refine(const int32_t* cand_idx, int32_t C, const void* q, li_dtype q_dt,
                       const float* w, const void* w_dec, li_dtype w_dt, const void* latent,
                       li_dtype c_dt, const float* c_scale, const int64_t* kv_off, int32_t B,
                       int32_t Gf, int32_t H, int32_t Dh, int32_t Dc, int32_t k, int32_t* out_idx,
                       float* out_scores, uint32_t flags, void* ws, size_t ws_bytes, void* stream);
size_t li_hs_refine_ws(int32_t B, int32_t C, int32_t Gf, int32_t H, int32_t Dc, int32_t k,
                       int32_t has_out_scores);

/* ---------------------------------------------------------------------------
 * li_latent_append — LatentIndex: write new tokens' rows of a group's shared
 * latent cache, built from the group's first-layer hidden states (LatentIndex
 * page, Abstract and Figure 1).  The page does not give the encoder; this is
 * the linear down-projection of Multi-head Latent Attention:
 *     latent[dst_row[m]][c] = bf16( sum_i h[m][i] * w_enc[c][i] )
 * accumulated in fp32 and rounded once to bfloat16 (nearest, ties to even).
 * A ragged batch appends each request's new tokens at rows of its own, e.g.
 * dst_row = kv_off[b] + old_len_b + j for its j-th new token.
 *
 *   h       [M][d_model]  LI_BF16, hidden states of the M new tokens
 *   w_enc   [Dc][d_model] LI_BF16
 *   dst_row [M] int64, device; each in [0, n_tok) and all distinct (a repeated
 *           row's contents are unspecified; the range is checked only under
 *           LI_DEBUG_VALIDATE)
 *   latent  [n_tok][Dc], written in place at the dst rows (other rows untouched):
 *           c_dt LI_BF16: bf16 (nearest even; c_scale unused, may be NULL);
 *           c_dt LI_FP8_E4M3: E4M3 codes, with c_scale [n_tok][ceil(Dc/128)] fp32 written
 *           too: per 128-value block of a row (the last one 64 values at Dc = 192),
 *           scale = the block's largest
 *           magnitude / 448 (1 for an all-zero block) and codes = E4M3 of
 *           value / scale, nearest even, saturating; all in fp32.  This is the
 *           fp8 latent li_latent_score_group and li_hs_refine read.
 *   M >= 0 (M = 0 does nothing; h and dst_row may then be NULL);
 *   d_model a positive multiple of 64;  Dc 128, 192 or 256
 *   ws      li_latent_append_ws(M, d_model, Dc, c_dt) bytes (fp32 partial sums
 *           of the K split; 0 for bf16 output when one split covers K)
 * ------------------------------------------------------------------------- */
li_status li_latent_append(const void* h, li_dtype h_dt, const void* w_enc, li_dtype w_dt,
                           const int64_t* dst_row, int32_t M, int32_t d_model, int32_t Dc, void* latent,
                           li_dtype c_dt, float* c_scale, int64_t n_tok, void* ws, size_t ws_bytes, void* stream);
size_t li_latent_append_ws(int32_t M, int32_t d_model, int32_t Dc, li_dtype c_dt);

/* ---------------------------------------------------------------------------
 * li_sparse_attention — the consumer of a selection: each request's heads
 * attend the cache rows its indexer kept.
 *
 * (IndexCache page, Symbol Map: the selected set holds the k positions sent to
 * core sparse attention.  "Multi-layer Indexer ...", The Brief: attention
 * consumes a selection, so an indexer on a second stream can run beside it.)
 * The pages do not give the attention; this is the latent decode attention of
 * their model: a cached row of Dk = 576 values per token, shared by all heads,
 * is the key and its first Dv = 512 values the value:
 *     out[b][h] = sum_j p_j kv[r_j][0:512] / sum_j p_j,  p_j = exp(s_j - max_j s_j),
 *     s_j = scale * (q[b][h] . kv[r_j]),  r_j = kv_off[b] + idx[b][j]
 * over the entries j with idx[b][j] >= 0.  A request with none gets out = 0.
 * Scores accumulate in fp32; p is rounded to bf16 for the value product and
 * for its sum.
 *
 *   q       [B][H][576] LI_BF16;  H a multiple of 64, at most 256
 *   kv      [n_tok][576] LI_BF16;  kv_off [B+1] int64, device
 *   idx     [B][k] int32, device: positions in [0, L_b), ascending, -1 padded
 *           (out_idx of li_index_decode); 1 <= k <= 65536
 *   out     [B][H][512] fp32
 *   ws      li_sparse_attention_ws(B, H, k) bytes (per-split partial outputs)
 * ------------------------------------------------------------------------- */
li_status li_sparse_attention(const void* q, li_dtype q_dt, const void* kv, li_dtype kv_dt, const int32_t* idx,
                              const int64_t* kv_off, int32_t B, int64_t n_tok, int32_t H, int32_t Dk, int32_t Dv,
                              int32_t k, float scale, float* out, void* ws, size_t ws_bytes, void* stream);
size_t li_sparse_attention_ws(int32_t B, int32_t H, int32_t k);

/* ---------------------------------------------------------------------------
 * Cache layouts in bytes per token (host only).  A key row of D values
 * (LI_FP8_E4M3: D bytes + one fp32 scale; LI_BF16: 2*D bytes) and a latent row
 * of Dc values (LI_FP8_E4M3: Dc bytes + one fp32 scale per started 128-value
 * block; LI_BF16: 2*Dc bytes).  LatentIndex page, Abstract: the shared latent
 * replaces per-layer indexer key caches.  0 for a dtype without a layout.
 * ------------------------------------------------------------------------- */
size_t li_key_row_bytes(int32_t D, li_dtype dt);
size_t li_latent_row_bytes(int32_t Dc, li_dtype dt);

/* ---------------------------------------------------------------------------
 * li_indexcache_plan — IndexCache layer roles (host only; no device work).
 *
 * ("IndexCache: Cross-Layer Index Reuse for Sparse Attention", Deep Dive and
 * its role table.)  A Full (F) layer runs its indexer and overwrites the index
 * buffer; a Shared (S) layer skips its indexer and attends the buffer left by
 * the nearest preceding F layer.  The first layer is always F.
 *
 *   roles    [n_layers] uint8, host: 1 = F, 0 = S; or NULL for the uniform
 *            pattern in which layer l is F when l % retain_every == 0 (retention
 *            1/retain_every, e.g. 4 gives F S S S F S S S ...)
 *   src      [n_layers] int32, host, written: the layer whose indexer produced
 *            the selection layer l attends (l itself for an F layer)
 *   returns  the number of F layers (indexer scans per token), or a negative
 *            li_status: -LI_E_NULL (src NULL), -LI_E_SHAPE (n_layers < 1,
 *            retain_every < 1 with roles NULL, or roles[0] not F)
 * ------------------------------------------------------------------------- */
int32_t li_indexcache_plan(const uint8_t* roles, int32_t n_layers, int32_t retain_every, int32_t* src);

/* ---------------------------------------------------------------------------
 * li_topk — the selection step on its own: per-row top-k of fp32 scores.
 *
 * Row r holds row_len[r] (or n, when row_len is NULL) scores at
 * scores + r * row_stride.  Keeps the k highest (ties: lower position; -0 == +0),
 * writes their positions ascending, -1 padded.  (IndexCache page, Deep Dive:
 * the indexer takes top-k of its scores to obtain the index tensor.)
 *
 *   scores [rows][row_stride] fp32; row_len [rows] int32 device or NULL,
 *   each 0 <= row_len[r] <= row_stride (not checked: device memory)
 *   0 <= n <= row_stride; 1 <= k <= LI_MAX_K; out_idx [rows][k] int32
 * ------------------------------------------------------------------------- */
li_status li_topk(const float* scores, int64_t row_stride, const int32_t* row_len, int32_t rows,
                  int32_t n, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream);
size_t li_topk_ws(int32_t rows, int32_t n, int32_t k);

/* ---------------------------------------------------------------------------
 * Measurement hook (not part of the computation): after li_trace_events(ev, n)
 * with n > 0, every entry point called on this thread launches its i-th
 * kernel (i = 0, 1, ...) with ev[2i] and ev[2i+1] as the launch's start and
 * stop events (hipExtLaunchKernel), which the runtime sets to that kernel's
 * own start and end, as long as pairs remain; hipEventElapsedTime(ev[2i],
 * ev[2i+1]) is then kernel i's duration.  li_trace_count() returns how many
 * events the last call used.  `events` are caller-created hipEvent_t handles
 * that must outlive their use.  li_trace_events(NULL, 0) switches the hook
 * off.
 * ------------------------------------------------------------------------- */
void li_trace_events(void** events, int32_t capacity);
int32_t li_trace_count(void);

/* Read-bandwidth probe (measurement aid, not part of the computation): one
 * kernel streams `bytes` bytes of `p` with the decode scan's load pattern
 * (16-byte non-temporal loads, 1 KB per wave per load, eight loads in flight
 * per lane) and folds the data into one word per wave of `sink`
 * (LI_READ_PROBE_SINK_WORDS uint32 words, device), so that its duration
 * (e.g. through li_trace_events) gives the read rate this GPU reaches for such
 * a stream.  p must be 16-byte
 * aligned and bytes a multiple of 16 (else LI_E_SHAPE). */
#define LI_READ_PROBE_SINK_WORDS 8192
li_status li_read_probe(const void* p, size_t bytes, uint32_t* sink, void* stream);

/* Matrix-core rate probe (measurement aid, not part of the computation): one
 * kernel of LI_MFMA_PROBE_WAVES waves (2048 workgroups of four, eight waves per
 * SIMD) in which every wave runs `iters` iterations of
 * LI_MFMA_PROBE_PRODUCTS_PER_ITER matrix products of one form, in two
 * independent accumulator chains over eight A and eight B operand registers:
 *   LI_MFMA_PROBE_F16   v_mfma_f32_16x16x32_f16       (16384 FLOP per product)
 *   LI_MFMA_PROBE_BF16  v_mfma_f32_32x32x16_bf16      (32768 FLOP)
 *   LI_MFMA_PROBE_FP8   v_mfma_f32_16x16x128_f8f6f4, E4M3 (65536 FLOP)
 * random_operands = 0 fills every operand element with 1.0, so that each
 * chain's accumulator grows by K (32, 16, 128) per product and sink word w
 * (one float per wave, LI_MFMA_PROBE_SINK_WORDS, device) is
 * 2 * 8 * K * iters exactly while that stays below 2^24; otherwise the
 * operands are pseudo-random values of the form (random signs and mantissas,
 * 16 octaves of exponents for fp16 / bf16, any finite E4M3 code).  clk
 * (LI_MFMA_PROBE_CLOCK_WORDS uint32 words, device) receives, per workgroup,
 * the shader clock cycles it ran (word 2i) and the 100 MHz real-time ticks it
 * ran (word 2i + 1), from which the shader clock follows.  The kernel's
 * duration (e.g. through li_trace_events) gives the product rate; the two
 * operand kinds bracket it, since the GPU lowers its clock under the power
 * drawn by products on varying data.  iters in [1, 2^20] and a known form,
 * else LI_E_SHAPE; null sink or clk: LI_E_NULL. */
#define LI_MFMA_PROBE_F16 0
#define LI_MFMA_PROBE_BF16 1
#define LI_MFMA_PROBE_FP8 2
#define LI_MFMA_PROBE_WAVES 8192
#define LI_MFMA_PROBE_PRODUCTS_PER_ITER 16
#define LI_MFMA_PROBE_SINK_WORDS 8192
#define LI_MFMA_PROBE_CLOCK_WORDS 4096
li_status li_mfma_probe(int32_t form, int32_t random_operands, int32_t iters, float* sink, uint32_t* clk,
                        void* stream);

/* Human-readable name of a status code (static storage). */
const char* li_status_str(li_status s);
/* Detail of the last error on this thread (e.g. the HIP error text); "" if none. */
const char* li_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LI_H */
