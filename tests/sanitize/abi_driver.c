/* Host-only driver of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * together with a host-sanitized build of the library (tests/test_abi_sanitized.py). It calls
 * every entry point with arguments that the library must reject, or that make the call a no-op,
 * so nothing reaches a GPU; the run fails on a wrong status or on any sanitizer report. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsa.h"

static int failures = 0;

#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    dsa_status_t st_ = (call);                                                                \
    if (st_ != (want)) {                                                                      \
      fprintf(stderr, "%s:%d: %s returned %d (%s: %s), expected %d\n", __FILE__, __LINE__,    \
              #call, (int)st_, dsa_status_string(st_), dsa_last_error(), (int)(want));       \
      ++failures;                                                                             \
    }                                                                                         \
  } while (0)

static _Alignas(16) unsigned char arena[4096];

static dsa_seqs_t make_seqs(const int32_t* cq, const int32_t* ck, int B, int max_m, int max_n) {
  dsa_seqs_t s;
  memset(&s, 0, sizeof s);
  s.num_seqs = B;
  s.cu_seqlens_q = cq;  /* never dereferenced by the host code */
  s.cu_seqlens_k = ck;
  s.cu_seqlens_q_host = cq;
  s.cu_seqlens_k_host = ck;
  s.max_seqlen_q = max_m;
  s.max_seqlen_k = max_n;
  return s;
}

int main(void) {
  void* p = arena;
  void* pm = arena + 4;   /* misaligned */
  const int32_t cq[] = {0, 3, 5}, ck[] = {0, 10, 16};
  dsa_seqs_t s = make_seqs(cq, ck, 2, 3, 10);

  /* sequence descriptions */
  EXPECT(dsa_indexer_scores(NULL, 64, 128, DSA_FP8_E4M3, p, p, p, p, 12, p, 0, NULL), DSA_ERR_NULL);
  dsa_seqs_t bad = make_seqs(cq, ck, 2, 3, 11);
  EXPECT(dsa_topk(&bad, p, 12, 4, p, NULL, 0, NULL), DSA_ERR_SHAPE);
  const int32_t cq2[] = {0, 12}, ck2[] = {0, 10};
  bad = make_seqs(cq2, ck2, 1, 12, 10);
  EXPECT(dsa_topk(&bad, p, 12, 4, p, NULL, 0, NULL), DSA_ERR_SHAPE);
  bad = s;
  bad.num_seqs = -3;
  EXPECT(dsa_topk(&bad, p, 12, 4, p, NULL, 0, NULL), DSA_ERR_SHAPE);
  bad = s;
  bad.cu_seqlens_k_host = NULL;
  EXPECT(dsa_topk(&bad, p, 12, 4, p, NULL, 0, NULL), DSA_ERR_NULL);
  const int32_t zero[] = {0};
  dsa_seqs_t empty = make_seqs(zero, zero, 0, 0, 0);
  EXPECT(dsa_topk(&empty, NULL, 4, 4, NULL, NULL, 0, NULL), DSA_OK);

  /* indexer */
  EXPECT(dsa_indexer_scores(&s, 64, 128, DSA_BF16, p, p, p, p, 12, p, 4096, NULL), DSA_ERR_DTYPE);
  EXPECT(dsa_indexer_scores(&s, 64, 128, (dsa_dtype_t)77, p, p, p, p, 12, p, 4096, NULL), DSA_ERR_DTYPE);
  if (dsa_indexer_workspace_size(&s, 64, 128, (dsa_dtype_t)-5) != 0) ++failures;
  EXPECT(dsa_indexer_scores(&s, 64, 128, DSA_FP8_E4M3, p, p, p, p, 10, p, 4096, NULL), DSA_ERR_SHAPE);
  EXPECT(dsa_indexer_scores(&s, 32, 128, DSA_FP8_E4M3, p, p, p, p, 12, p, 4096, NULL), DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_indexer_scores(&s, 64, 128, DSA_FP8_E4M3, p, NULL, p, p, 12, p, 4096, NULL), DSA_ERR_NULL);
  EXPECT(dsa_indexer_scores(&s, 64, 128, DSA_FP8_E4M3, p, p, pm, p, 12, p, 4096, NULL), DSA_ERR_ALIGN);
  size_t need = dsa_indexer_workspace_size(&s, 64, 128, DSA_FP8_E4M3);
  if (need < 5 * 516) { fprintf(stderr, "indexer workspace %zu too small\n", need); ++failures; }
  EXPECT(dsa_indexer_scores(&s, 64, 128, DSA_FP8_E4M3, p, p, p, p, 12, p, need - 1, NULL), DSA_ERR_WORKSPACE);
  EXPECT(dsa_indexer_scores_scaled(&s, 64, 128, DSA_FP8_E4M3, p, pm, p, p, p, p, 12, p, 1 << 20, NULL),
         DSA_ERR_ALIGN);
  EXPECT(dsa_indexer_scores_scaled(&s, 64, 128, DSA_FP8_E4M3, p, p, p, p, p, p, 12, NULL, 0, NULL),
         DSA_ERR_WORKSPACE);
  if (dsa_indexer_scaled_workspace_size(&s, 64, 128, DSA_FP8_E4M3) < need) ++failures;

  /* top-k */
  EXPECT(dsa_topk(&s, p, 12, 0, p, NULL, 0, NULL), DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_topk(&s, p, 12, 16385, p, NULL, 0, NULL), DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_topk(&s, p, 14, 4, p, NULL, 0, NULL), DSA_ERR_SHAPE);
  EXPECT(dsa_topk(&s, p, 12, 4, pm, NULL, 0, NULL), DSA_ERR_ALIGN);
  (void)dsa_topk_workspace_size(&s, 2048);

  /* attention */
  EXPECT(dsa_sparse_mla_attn(&s, 128, 576, 512, DSA_FP8_E4M3, p, p, p, 64, 0.04f, p, p, NULL, 0, NULL),
         DSA_ERR_DTYPE);
  EXPECT(dsa_sparse_mla_attn(&s, 128, 576, 512, (dsa_dtype_t)9, p, p, p, 64, 0.04f, p, p, NULL, 0, NULL),
         DSA_ERR_DTYPE);
  EXPECT(dsa_sparse_mla_attn(&s, 128, 576, 600, DSA_BF16, p, p, p, 64, 0.04f, p, p, NULL, 0, NULL),
         DSA_ERR_SHAPE);
  EXPECT(dsa_sparse_mla_attn(&s, 64, 576, 512, DSA_BF16, p, p, p, 64, 0.04f, p, p, NULL, 0, NULL),
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_sparse_mla_attn(&s, 128, 576, 512, DSA_BF16, p, p, p, 64, -1.0f, p, p, NULL, 0, NULL),
         DSA_ERR_SHAPE);
  const int32_t cqd[] = {0, 1, 2}, ckd[] = {0, 4000, 9000};
  dsa_seqs_t dec = make_seqs(cqd, ckd, 2, 1, 5000);
  size_t aws = dsa_sparse_mla_attn_workspace_size(&dec, 128, 576, 512, 2048, DSA_BF16);
  if (aws == 0) { fprintf(stderr, "decode attention needs split workspace\n"); ++failures; }
  EXPECT(dsa_sparse_mla_attn(&dec, 128, 576, 512, DSA_BF16, p, p, p, 2048, 0.04f, p, p, p, aws - 1, NULL),
         DSA_ERR_WORKSPACE);

  /* fused forward */
  dsa_forward_args_t a;
  memset(&a, 0, sizeof a);
  a.H_I = 64; a.d_I = 128; a.qk_dtype = DSA_FP8_E4M3; a.q_idx = a.k_idx = p; a.w = (const float*)p;
  a.k = 4; a.H = 128; a.d_qk = 576; a.d_v = 512; a.dtype = DSA_BF16; a.q = a.kv = p; a.out = p;
  a.lse = (float*)p; a.softmax_scale = 0.04f;
  size_t fws = dsa_forward_workspace_size(&s, &a);
  EXPECT(dsa_forward(&s, &a, NULL, 0, NULL), DSA_ERR_WORKSPACE);
  EXPECT(dsa_forward(&s, &a, p, fws - 1, NULL), DSA_ERR_WORKSPACE);
  EXPECT(dsa_forward(&s, NULL, p, fws, NULL), DSA_ERR_NULL);
  a.softmax_scale = 0.0f;
  EXPECT(dsa_forward(&s, &a, p, fws, NULL), DSA_ERR_SHAPE);
  if (dsa_forward_workspace_size(NULL, &a) != 0 || dsa_forward_workspace_size(&s, NULL) != 0) ++failures;
  /* the no-allocation variant rejects a batch beyond its scratch before touching a device */
  const int32_t cqp[] = {0, 6000}, ckp[] = {0, 6000};
  dsa_seqs_t pre = make_seqs(cqp, ckp, 1, 6000, 6000);
  a.softmax_scale = 0.04f;
  a.k = 2048;
  if (dsa_forward_workspace_size(&pre, &a) <= DSA_NOALLOC_SCRATCH_BYTES) ++failures;
  EXPECT(dsa_forward_noalloc(&pre, &a, NULL), DSA_ERR_WORKSPACE);
  EXPECT(dsa_forward_noalloc(&pre, NULL, NULL), DSA_ERR_NULL);
  EXPECT(dsa_forward_noalloc(&empty, &a, NULL), DSA_OK);

  /* alignment target */
  EXPECT(dsa_indexer_alignment(&s, 128, 576, DSA_F32, p, p, p, 64, 0.04f, (const float*)p, (const float*)p,
                               12, NULL, (float*)p, NULL),
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_indexer_alignment(&s, 128, 576, DSA_BF16, p, p, p, 64, 0.04f, NULL, (const float*)p, 12, NULL,
                               (float*)p, NULL),
         DSA_ERR_NULL);

  /* status strings, last error, version */
  for (int st = -2; st < 10; ++st)
    if (!dsa_status_string((dsa_status_t)st)) ++failures;
  if (strcmp(dsa_status_string((dsa_status_t)1000), "unknown status") != 0) ++failures;
  if (dsa_abi_version() != DSA_ABI_VERSION) ++failures;
  if (strlen(dsa_last_error()) >= 512) ++failures;

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi driver: all checks passed\n");
  return 0;
}
