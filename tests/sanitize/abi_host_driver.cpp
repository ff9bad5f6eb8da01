// Host sanitizer driver for the C ABI (test infrastructure).
//
// Built from the library's sources with only their host side compiled, under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py),
// and run without a GPU: every call here is one the library must answer on
// the host, before any device work (argument and workspace checks, workspace
// size queries over extreme shapes, the IndexCache planner, row-size queries,
// status strings, the trace hook's bookkeeping).  A pointer that is never
// dereferenced stands in for device buffers.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "li.h"

static int fails = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const li_status got_ = (call);                                                          \
    if (got_ != (want)) {                                                                   \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, \
              (int)(want), li_last_error());                                                \
      ++fails;                                                                              \
    }                                                                                       \
  } while (0)

int main() {
  void* F = reinterpret_cast<void*>(uintptr_t(0x1000));
  const float* Ff = static_cast<const float*>(F);
  const int64_t* Fo = static_cast<const int64_t*>(F);
  int32_t* Fi = static_cast<int32_t*>(F);
  const size_t big = (size_t)1 << 40;

  // workspace queries over small, zero, negative and large shapes
  const int32_t Bs[] = {-1, 0, 1, 32, 4096};
  const int64_t Ns[] = {-5, 0, 1, 1 << 20, (int64_t)1 << 33};
  const int32_t ks[] = {1, 2048, LI_MAX_K};
  for (int32_t B : Bs)
    for (int64_t n : Ns)
      for (int32_t k : ks) {
        (void)li_index_decode_ws(B, n, (int32_t)(n > 0 && n < (1 << 30) ? n : 1), k, 0);
        (void)li_index_decode_ws(B, n, 131072, k, 1);
        (void)li_latent_score_group_ws(B, n, 131072, 4, 64, 256, k, 0);
        (void)li_hs_refine_ws(B, 8192, 3, 64, 256, k, 0);
        (void)li_index_prefill_ws(B, (int32_t)(n > 0 && n < (1 << 30) ? n : 0), k, 0);
        (void)li_sparse_attention_ws(B, 128, k);
        (void)li_latent_append_ws(B, 7168, 256, LI_FP8_E4M3);
        (void)li_topk_ws(B, 1000, k);
      }

  // decode
  EXPECT(li_index_decode(nullptr, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, 100, 60, 64, 128, 16, Fi, nullptr,
                         F, big, nullptr), LI_E_NULL);
  EXPECT(li_index_decode(F, LI_FP16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, 100, 60, 64, 128, 16, Fi, nullptr, F, big,
                         nullptr), LI_E_DTYPE);
  EXPECT(li_index_decode(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, 100, 60, 65, 128, 16, Fi, nullptr, F, big,
                         nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_index_decode(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, 100, 60, 64, 128, 0, Fi, nullptr, F, big,
                         nullptr), LI_E_SHAPE);
  EXPECT(li_index_decode(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, 100, 60, 64, 128, 16, Fi, nullptr, F, 8,
                         nullptr), LI_E_WORKSPACE);
  EXPECT(li_index_decode(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 0, 100, 60, 64, 128, 16, Fi, nullptr, F, big,
                         nullptr), LI_OK);
  EXPECT(li_index_decode_noalloc(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 2, (int64_t)1 << 25, 1 << 22, 64, 128,
                                 16, Fi, nullptr, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_index_decode_noalloc(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 64, (int64_t)64 << 17, 1 << 17, 64,
                                 128, 16, Fi, nullptr, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_index_decode_noalloc(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 0, 100, 60, 64, 128, 16, Fi, nullptr,
                                 nullptr), LI_OK);
  // prefill
  EXPECT(li_index_prefill(F, LI_FP8_E4M3, nullptr, Ff, F, LI_FP8_E4M3, nullptr, 10, 100, 91, 64, 128, 5, Fi,
                          nullptr, F, big, nullptr), LI_E_SHAPE);
  EXPECT(li_index_prefill(F, LI_FP8_E4M3, nullptr, Ff, F, LI_FP8_E4M3, nullptr, 10, 100, 90, 4, 128, 5, Fi,
                          nullptr, F, big, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_index_prefill(F, LI_FP8_E4M3, nullptr, Ff, F, LI_FP8_E4M3, nullptr, 0, 100, 0, 64, 128, 5, Fi,
                          nullptr, F, big, nullptr), LI_OK);
  // latent and HS
  EXPECT(li_latent_score_group(F, LI_BF16, Ff, F, LI_BF16, F, LI_BF16, nullptr, Fo, 2, 1000, 600, 4, 64, 128, 160,
                               8, Fi, nullptr, 0, F, big, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_latent_score_group(F, LI_BF16, Ff, F, LI_BF16, F, LI_FP8_E4M3, nullptr, Fo, 2, 1000, 600, 4, 64, 128,
                               256, 8, Fi, nullptr, 0, F, big, nullptr), LI_E_NULL);
  EXPECT(li_latent_score_group(F, LI_BF16, Ff, F, LI_BF16, F, LI_BF16, nullptr, Fo, 2, 1000, 600, 4, 1, 128, 256, 8,
                               Fi, nullptr, 0, F, big, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_latent_score_group(F, LI_BF16, Ff, F, LI_BF16, F, LI_BF16, nullptr, Fo, 0, 1000, 600, 4, 64, 128, 256, 8,
                               Fi, nullptr, 0, F, big, nullptr), LI_OK);
  EXPECT(li_hs_refine(static_cast<const int32_t*>(F), 70000, F, LI_BF16, Ff, F, LI_BF16, F, LI_BF16, nullptr, Fo, 1,
                      3, 64, 128, 256, 16, Fi, nullptr, 0, F, big, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_hs_refine(static_cast<const int32_t*>(F), 8192, F, LI_BF16, Ff, F, LI_BF16, F, LI_BF16, nullptr, Fo, 0,
                      3, 64, 128, 256, 16, Fi, nullptr, 0, F, big, nullptr), LI_OK);
  // append, attention, top-k
  EXPECT(li_latent_append(F, LI_BF16, F, LI_BF16, Fo, 4, 7168 + 32, 256, F, LI_BF16, nullptr, 100, F, big, nullptr),
         LI_E_UNSUPPORTED);
  EXPECT(li_latent_append(F, LI_BF16, F, LI_BF16, Fo, 0, 7168, 256, F, LI_BF16, nullptr, 100, nullptr, 0, nullptr),
         LI_OK);
  EXPECT(li_sparse_attention(F, LI_BF16, F, LI_BF16, Fi, Fo, 2, 100, 96, 576, 512, 2048, 0.1f, static_cast<float*>(F),
                             F, big, nullptr), LI_E_UNSUPPORTED);
  EXPECT(li_topk(Ff, 5, nullptr, 1, 10, 1, Fi, F, big, nullptr), LI_E_SHAPE);
  EXPECT(li_topk(Ff, 10, nullptr, 0, 10, 3, Fi, F, big, nullptr), LI_OK);
  EXPECT(li_read_probe(F, 1000, static_cast<uint32_t*>(F), nullptr), LI_E_SHAPE);
  EXPECT(li_mfma_probe(LI_MFMA_PROBE_F16, 0, 16, nullptr, static_cast<uint32_t*>(F), nullptr), LI_E_NULL);
  EXPECT(li_mfma_probe(3, 1, 16, static_cast<float*>(F), static_cast<uint32_t*>(F), nullptr), LI_E_SHAPE);
  EXPECT(li_mfma_probe(LI_MFMA_PROBE_FP8, 1, 0, static_cast<float*>(F), static_cast<uint32_t*>(F), nullptr), LI_E_SHAPE);

  // IndexCache planner (host only)
  int32_t src[61];
  if (li_indexcache_plan(nullptr, 61, 4, src) != 16) ++fails;
  uint8_t roles[61];
  for (int l = 0; l < 61; ++l) roles[l] = (uint8_t)(l % 3 == 0);
  if (li_indexcache_plan(roles, 61, 0, src) != 21) ++fails;
  if (li_indexcache_plan(nullptr, 0, 4, src) != -LI_E_SHAPE) ++fails;
  if (li_indexcache_plan(nullptr, 61, 4, nullptr) != -LI_E_NULL) ++fails;

  // row sizes, status strings, trace bookkeeping
  if (li_latent_row_bytes(256, LI_FP8_E4M3) != 264 || li_key_row_bytes(128, LI_FP8_E4M3) != 132) ++fails;
  for (int s = -1; s < 10; ++s)
    if (!li_status_str(s) || !strlen(li_status_str(s))) ++fails;
  void* ev[4] = {nullptr, nullptr, nullptr, nullptr};
  li_trace_events(ev, 4);
  EXPECT(li_index_decode(F, LI_BF16, Ff, F, LI_FP8_E4M3, nullptr, Fo, 0, 100, 60, 64, 128, 16, Fi, nullptr, F, big,
                         nullptr), LI_OK);
  if (li_trace_count() != 0) ++fails;
  li_trace_events(nullptr, 0);

  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("abi host driver ok\n");
  return 0;
}
