// Host side of the C ABI declared in include/dsa.h: argument validation (before anything is
// enqueued), dispatch to the kernels, workspace planning.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "dsa_internal.h"

namespace {

thread_local char g_err[512] = "";

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

dsa_status_t ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Validates a sequence description and fills the launch-planning summary.
dsa_status_t check_seqs(const dsa_seqs_t* s, dsa::SeqInfo& info) {
  if (!s) return fail(DSA_ERR_NULL, "seqs is NULL");
  if (s->num_seqs < 0) return fail(DSA_ERR_SHAPE, "num_seqs = %d < 0", s->num_seqs);
  info = dsa::SeqInfo{};
  info.B = s->num_seqs;
  if (s->num_seqs == 0) return ok();
  if (!s->cu_seqlens_q || !s->cu_seqlens_k)
    return fail(DSA_ERR_NULL, "device cu_seqlens pointer is NULL");
  if (!s->cu_seqlens_q_host || !s->cu_seqlens_k_host)
    return fail(DSA_ERR_NULL, "host cu_seqlens pointer is NULL");
  const int32_t* cq = s->cu_seqlens_q_host;
  const int32_t* ck = s->cu_seqlens_k_host;
  if (cq[0] != 0 || ck[0] != 0) return fail(DSA_ERR_SHAPE, "cu_seqlens must start at 0");
  int max_m = 0, max_n = 0;
  for (int b = 0; b < s->num_seqs; ++b) {
    const int64_t m = (int64_t)cq[b + 1] - cq[b], n = (int64_t)ck[b + 1] - ck[b];
    if (m < 0 || n < 0) return fail(DSA_ERR_SHAPE, "cu_seqlens decrease at sequence %d", b);
    if (m > n) return fail(DSA_ERR_SHAPE, "sequence %d has %lld queries but %lld keys", b,
                           (long long)m, (long long)n);
    if (m > max_m) max_m = (int)m;
    if (n > max_n) max_n = (int)n;
  }
  if (max_m != s->max_seqlen_q || max_n != s->max_seqlen_k)
    return fail(DSA_ERR_SHAPE, "max_seqlen_q/k (%d, %d) differ from the true maxima (%d, %d)",
                s->max_seqlen_q, s->max_seqlen_k, max_m, max_n);
  info.T = cq[s->num_seqs];
  info.Nk = ck[s->num_seqs];
  info.max_m = max_m;
  info.max_n = max_n;
  info.cu_q = s->cu_seqlens_q;
  info.cu_k = s->cu_seqlens_k;
  info.cu_q_host = cq;
  info.cu_k_host = ck;
  return ok();
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// `scores` is only checked when `own_scores` is false (dsa_forward places it in the workspace).
dsa_status_t check_indexer(const dsa::SeqInfo& s, int32_t H_I, int32_t d_I, dsa_dtype_t dt,
                           const void* q, const void* k, const float* w, const float* scores,
                           int64_t ld, bool own_scores = false) {
  if (dt != DSA_FP8_E4M3 && dt != DSA_F32)
    return fail(DSA_ERR_DTYPE, "indexer inputs must be DSA_FP8_E4M3 or DSA_F32");
  if (H_I <= 0 || d_I <= 0) return fail(DSA_ERR_SHAPE, "H_I and d_I must be positive");
  if (ld < s.max_n || ld % 4 != 0)
    return fail(DSA_ERR_SHAPE, "ld_scores = %lld must be >= max_seqlen_k (%d) and a multiple of 4",
                (long long)ld, s.max_n);
  if (s.T == 0) return ok();
  if (!q || !k || !w || (!scores && !own_scores))
    return fail(DSA_ERR_NULL, "indexer tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(w) || (scores && !aligned16(scores)))
    return fail(DSA_ERR_ALIGN, "indexer tensors must be 16-byte aligned");
  if (dt == DSA_FP8_E4M3 && !(H_I == 64 && d_I == 128))
    return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer needs H_I = 64, d_I = 128 (got %d, %d)", H_I, d_I);
  if (dt == DSA_FP8_E4M3 && (int64_t)s.max_n * d_I > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer needs max_seqlen_k * 128 < 2^31 (got %d keys)", s.max_n);
  if (dt == DSA_F32 && (H_I > 128 || d_I > 256 || H_I * d_I > 16384))
    return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer supports H_I <= 128, d_I <= 256, H_I*d_I <= 16384");
  // launch grids: the FP8 kernels give each sequence a grid layer, the fp32 kernel each 256-key
  // slice of a row, and those grid dimensions hold at most 65535
  if (dt == DSA_FP8_E4M3 && s.B > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "FP8 indexer takes at most 65535 sequences per call (got %d)", s.B);
  if (dt == DSA_F32 && (s.max_n + 255) / 256 > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer takes at most 65535 * 256 keys per sequence (got %d)",
                s.max_n);
  return ok();
}

dsa_status_t check_topk(const dsa::SeqInfo& s, const float* scores, int64_t ld, int32_t k,
                        const int32_t* idx) {
  if (k < 1 || k > 16384) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside 1..16384", k);
  if (ld < s.max_n || ld % 4 != 0)
    return fail(DSA_ERR_SHAPE, "ld_scores = %lld must be >= max_seqlen_k (%d) and a multiple of 4",
                (long long)ld, s.max_n);
  if (s.T == 0) return ok();
  if (!scores || !idx) return fail(DSA_ERR_NULL, "scores or indices is NULL");
  if (!aligned16(scores) || !aligned16(idx))
    return fail(DSA_ERR_ALIGN, "scores and indices must be 16-byte aligned");
  return ok();
}

// `idx` is only checked when `own_idx` is false (dsa_forward places it in the workspace).
dsa_status_t check_attn(const dsa::SeqInfo& s, int32_t H, int32_t d_qk, int32_t d_v,
                        dsa_dtype_t dt, const void* q, const void* kv, const int32_t* idx,
                        int32_t k, const void* out, const float* lse, bool own_idx = false) {
  if (dt != DSA_BF16 && dt != DSA_F32)
    return fail(DSA_ERR_DTYPE, "attention inputs must be DSA_BF16 or DSA_F32");
  if (H <= 0 || d_qk <= 0 || d_v <= 0) return fail(DSA_ERR_SHAPE, "H, d_qk, d_v must be positive");
  if (d_v > d_qk) return fail(DSA_ERR_SHAPE, "d_v = %d exceeds d_qk = %d", d_v, d_qk);
  if (k < 1 || k > 16384) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside 1..16384", k);
  if (s.T == 0) return ok();
  if (!q || !kv || (!idx && !own_idx) || !out)
    return fail(DSA_ERR_NULL, "attention tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(kv) || (idx && !aligned16(idx)) || !aligned16(out) ||
      (lse && !aligned16(lse)))
    return fail(DSA_ERR_ALIGN, "attention tensors must be 16-byte aligned");
  if (dt == DSA_BF16 && !(H == 128 && d_qk == 576 && d_v == 512))
    return fail(DSA_ERR_UNSUPPORTED, "bf16 attention needs (H, d_qk, d_v) = (128, 576, 512)");
  if (dt == DSA_BF16 && (int64_t)s.max_n * d_qk * 2 > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "bf16 attention needs max_seqlen_k * 1152 < 2^31 (got %d keys)",
                s.max_n);
  if (dt == DSA_F32 && (H > 128 || d_qk > 1024 || k > 4096))
    return fail(DSA_ERR_UNSUPPORTED, "fp32 attention supports H <= 128, d_qk <= 1024, k <= 4096");
  return ok();
}

// Bytes of indexer workspace: the FP8 prefill path keeps per-row data of the query side there;
// with query scales, the scaled head weights [T, H_I] follow.
size_t indexer_ws_bytes(const dsa::SeqInfo& s, dsa_dtype_t dt) {
  return (dt == DSA_FP8_E4M3 && s.max_m > 1) ? dsa::indexer_workspace_bytes(s, true) : 0;
}
size_t indexer_scaled_ws_bytes(const dsa::SeqInfo& s, int32_t H_I, dsa_dtype_t dt) {
  return align_up(indexer_ws_bytes(s, dt)) + align_up((size_t)s.T * H_I * sizeof(float));
}

// The fused indexer -> top-k takes the fused path (chunk candidates + merge) for FP8 decode
// batches; its workspace is the indexer's, then the candidates or the top-k's.
bool indexer_topk_fused(const dsa::SeqInfo& s, int32_t H_I, int32_t d_I, dsa_dtype_t dt, int32_t k) {
  return dt == DSA_FP8_E4M3 && H_I == 64 && d_I == 128 && dsa::decode_fused_topk_ok(s, k);
}
size_t indexer_topk_ws_bytes(const dsa::SeqInfo& s, int32_t H_I, int32_t d_I, dsa_dtype_t dt, int32_t k) {
  return align_up(indexer_ws_bytes(s, dt)) +
         (indexer_topk_fused(s, H_I, d_I, dt, k) ? dsa::decode_cand_bytes(s, k) : dsa::topk_workspace_bytes(s, k));
}

// qscale [T, H_I] / kscale [Nk]: optional positive scales of the indexer queries and keys.
// cand: the fused decode top-k's candidate buffers (FP8 decode batches only), or NULL.
dsa_status_t run_indexer(const dsa::SeqInfo& s, int32_t H_I, int32_t d_I, dsa_dtype_t dt,
                         const void* q, const float* qscale, const void* k, const float* kscale,
                         const float* w, float* scores, int64_t ld, void* ws, hipStream_t st,
                         const dsa::DecodeCand* cand = nullptr) {
  if (s.T == 0) return ok();
  hipError_t e;
  if (qscale) {   // fold the query scales into the head weights
    float* weff = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(indexer_ws_bytes(s, dt)));
    e = dsa::launch_indexer_scale_weights(s, H_I, w, qscale, weff, st);
    if (e != hipSuccess) return hip_status(e, "indexer scale launch");
    w = weff;
  }
  if (dt == DSA_F32)
    e = dsa::launch_indexer_f32(s, H_I, d_I, static_cast<const float*>(q),
                                static_cast<const float*>(k), w, kscale, scores, ld, st);
  else if (s.max_m == 1)
    e = dsa::launch_indexer_fp8_decode(s, static_cast<const uint8_t*>(q),
                                       static_cast<const uint8_t*>(k), w, kscale, scores, ld, cand, st);
  else
    e = dsa::launch_indexer_fp8_prefill(s, static_cast<const uint8_t*>(q),
                                        static_cast<const uint8_t*>(k), w, kscale, scores, ld, ws,
                                        st);
  return hip_status(e, "indexer launch");
}

// prefix_rows: idx was written by this library's top-k in the same call (see launch_attn_bf16).
dsa_status_t run_attn(const dsa::SeqInfo& s, int32_t H, int32_t d_qk, int32_t d_v, dsa_dtype_t dt,
                      const void* q, const void* kv, const int32_t* idx, int32_t k, float scale,
                      void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st,
                      bool prefix_rows = false) {
  if (s.T == 0) return ok();
  hipError_t e;
  if (dt == DSA_F32)
    e = dsa::launch_attn_f32(s, H, d_qk, d_v, static_cast<const float*>(q),
                             static_cast<const float*>(kv), idx, k, scale,
                             static_cast<float*>(out), lse, st);
  else
    e = dsa::launch_attn_bf16(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv),
                              idx, k, scale, static_cast<uint16_t*>(out), lse, ws, ws_bytes, prefix_rows,
                              st);
  return hip_status(e, "attention launch");
}

struct ForwardPlan {
  int64_t ld;
  bool dense, run_indexer, implicit_idx, run_topk;
  size_t index_off, index_bytes;
  size_t scores_off, scores_bytes;
  size_t idx_off, idx_bytes;
  size_t topk_off, topk_bytes;
  size_t attn_off, attn_bytes;
  size_t total;
};

// Row stride of the scores the fused call keeps in its workspace: max_seqlen_k rounded up to 4.
int64_t default_ld(const dsa::SeqInfo& s) { return std::max<int64_t>(4, ((int64_t)s.max_n + 3) / 4 * 4); }

ForwardPlan plan_forward(const dsa::SeqInfo& s, const dsa_forward_args_t* a) {
  ForwardPlan p{};
  p.ld = default_ld(s);
  // Short contexts: with at most k keys per sequence every row selects all its candidates, so
  // the scores are only computed when the caller asks for them, and the bf16 attention walks the
  // candidates without an index list (top-k only runs to fill indices_out, or for the fp32 path).
  p.dense = s.max_n <= a->k;
  p.run_indexer = !p.dense || a->scores_out != nullptr;
  p.implicit_idx = p.dense && a->dtype == DSA_BF16;
  p.run_topk = !p.implicit_idx || a->indices_out != nullptr;
  size_t off = 0;
  p.index_bytes = !p.run_indexer ? 0
                  : (a->q_idx_scale ? indexer_scaled_ws_bytes(s, a->H_I, a->qk_dtype)
                                    : align_up(indexer_ws_bytes(s, a->qk_dtype)));
  p.index_off = off;
  off += p.index_bytes;
  p.scores_bytes = (a->scores_out || p.dense) ? 0 : align_up((size_t)s.T * p.ld * sizeof(float));
  p.scores_off = off;
  off += p.scores_bytes;
  p.idx_bytes = (a->indices_out || !p.run_topk) ? 0 : align_up((size_t)s.T * a->k * sizeof(int32_t));
  p.idx_off = off;
  off += p.idx_bytes;
  p.topk_bytes = p.run_topk ? align_up(dsa::topk_workspace_bytes(s, a->k)) : 0;
  p.topk_off = off;
  off += p.topk_bytes;
  p.attn_bytes = align_up(dsa::attn_workspace_bytes(s, a->H, a->d_qk, a->d_v, a->k, a->dtype == DSA_BF16));
  p.attn_off = off;
  off += p.attn_bytes;
  p.total = off;
  return p;
}

// Argument checks of the fused call, before any workspace planning (the plan's sizes assume them).
dsa_status_t check_forward(const dsa::SeqInfo& s, const dsa_forward_args_t* a) {
  const int64_t ld = a->scores_out ? a->ld_scores_out : default_ld(s);
  dsa_status_t st = check_indexer(s, a->H_I, a->d_I, a->qk_dtype, a->q_idx, a->k_idx, a->w, a->scores_out,
                                  ld, a->scores_out == nullptr);
  if (st != DSA_OK) return st;
  st = check_attn(s, a->H, a->d_qk, a->d_v, a->dtype, a->q, a->kv, a->indices_out, a->k, a->out,
                  a->lse, a->indices_out == nullptr);
  if (st != DSA_OK) return st;
  if (!(a->softmax_scale > 0.f) || a->softmax_scale > 3.0e38f)
    return fail(DSA_ERR_SHAPE, "softmax_scale must be positive and finite (got %g)", a->softmax_scale);
  if ((a->q_idx_scale && !aligned16(a->q_idx_scale)) || (a->k_idx_scale && !aligned16(a->k_idx_scale)))
    return fail(DSA_ERR_ALIGN, "scale arrays must be 16-byte aligned");
  return ok();
}

// ---------------------------------------------------------------- scratch of dsa_forward_noalloc
// One static device array per GPU (each device that loads the library holds its own copy until
// the process ends). In host code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is ever
// passed to kernels.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace


extern "C" {

size_t dsa_indexer_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                  dsa_dtype_t qk_dtype) {
  dsa::SeqInfo s;
  if (check_seqs(seqs, s) != DSA_OK || s.B == 0 || H_I <= 0 || d_I <= 0) return 0;
  return indexer_ws_bytes(s, qk_dtype);
}

dsa_status_t dsa_indexer_scores(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                dsa_dtype_t qk_dtype, const void* q_idx, const void* k_idx,
                                const float* w, float* scores, int64_t ld_scores, void* ws,
                                size_t ws_bytes, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  st = check_indexer(s, H_I, d_I, qk_dtype, q_idx, k_idx, w, scores, ld_scores);
  if (st != DSA_OK) return st;
  const size_t need = indexer_ws_bytes(s, qk_dtype);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "indexer workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return run_indexer(s, H_I, d_I, qk_dtype, q_idx, nullptr, k_idx, nullptr, w, scores, ld_scores, ws,
                     static_cast<hipStream_t>(stream));
}

size_t dsa_indexer_scaled_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                         dsa_dtype_t qk_dtype) {
  dsa::SeqInfo s;
  if (check_seqs(seqs, s) != DSA_OK || s.B == 0 || H_I <= 0 || d_I <= 0) return 0;
  return indexer_scaled_ws_bytes(s, H_I, qk_dtype);
}

dsa_status_t dsa_indexer_scores_scaled(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                       dsa_dtype_t qk_dtype, const void* q_idx, const float* q_scale,
                                       const void* k_idx, const float* k_scale, const float* w,
                                       float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                                       void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  st = check_indexer(s, H_I, d_I, qk_dtype, q_idx, k_idx, w, scores, ld_scores);
  if (st != DSA_OK) return st;
  if ((q_scale && !aligned16(q_scale)) || (k_scale && !aligned16(k_scale)))
    return fail(DSA_ERR_ALIGN, "scale arrays must be 16-byte aligned");
  const size_t need = indexer_scaled_ws_bytes(s, H_I, qk_dtype);
  if (s.T > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "scaled indexer workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return run_indexer(s, H_I, d_I, qk_dtype, q_idx, q_scale, k_idx, k_scale, w, scores, ld_scores,
                     ws, static_cast<hipStream_t>(stream));
}

size_t dsa_topk_workspace_size(const dsa_seqs_t* seqs, int32_t k) {
  dsa::SeqInfo s;
  if (check_seqs(seqs, s) != DSA_OK || s.B == 0 || k < 1) return 0;
  return dsa::topk_workspace_bytes(s, k);
}

dsa_status_t dsa_topk(const dsa_seqs_t* seqs, const float* scores, int64_t ld_scores, int32_t k,
                      int32_t* indices, void* ws, size_t ws_bytes, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  st = check_topk(s, scores, ld_scores, k, indices);
  if (st != DSA_OK) return st;
  const size_t need = dsa::topk_workspace_bytes(s, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (s.T == 0) return ok();
  return hip_status(dsa::launch_topk(s, scores, ld_scores, k, indices, ws, ws_bytes,
                                     static_cast<hipStream_t>(stream)),
                    "top-k launch");
}

size_t dsa_indexer_topk_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                       dsa_dtype_t qk_dtype, int32_t k) {
  dsa::SeqInfo s;
  if (check_seqs(seqs, s) != DSA_OK || s.B == 0 || H_I <= 0 || d_I <= 0 || k < 1) return 0;
  return indexer_topk_ws_bytes(s, H_I, d_I, qk_dtype, k);
}

dsa_status_t dsa_indexer_topk(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I, dsa_dtype_t qk_dtype,
                              const void* q_idx, const void* k_idx, const float* w, float* scores,
                              int64_t ld_scores, int32_t k, int32_t* indices, void* ws, size_t ws_bytes,
                              void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  st = check_indexer(s, H_I, d_I, qk_dtype, q_idx, k_idx, w, scores, ld_scores);
  if (st != DSA_OK) return st;
  st = check_topk(s, scores, ld_scores, k, indices);
  if (st != DSA_OK) return st;
  const size_t need = indexer_topk_ws_bytes(s, H_I, d_I, qk_dtype, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "indexer top-k workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (ws && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DSA_ERR_ALIGN, "indexer top-k workspace must be %zu-byte aligned", kAlign);
  if (s.T == 0) return ok();
  char* base = static_cast<char*>(ws);
  const size_t iws = align_up(indexer_ws_bytes(s, qk_dtype));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (indexer_topk_fused(s, H_I, d_I, qk_dtype, k)) {
    const dsa::DecodeCand cand = dsa::decode_cand_layout(s, k, base + iws);
    st = run_indexer(s, H_I, d_I, qk_dtype, q_idx, nullptr, k_idx, nullptr, w, scores, ld_scores,
                     iws ? base : nullptr, hs, &cand);
    if (st != DSA_OK) return st;
    return hip_status(dsa::launch_topk_merge_decode(s, scores, ld_scores, k, indices, cand, hs),
                      "top-k merge launch");
  }
  st = run_indexer(s, H_I, d_I, qk_dtype, q_idx, nullptr, k_idx, nullptr, w, scores, ld_scores,
                   iws ? base : nullptr, hs);
  if (st != DSA_OK) return st;
  const size_t tws = dsa::topk_workspace_bytes(s, k);
  return hip_status(dsa::launch_topk(s, scores, ld_scores, k, indices, tws ? base + iws : nullptr, tws, hs),
                    "top-k launch");
}

size_t dsa_sparse_mla_attn_workspace_size(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk,
                                          int32_t d_v, int32_t k, dsa_dtype_t dtype) {
  dsa::SeqInfo s;
  if (check_seqs(seqs, s) != DSA_OK || s.B == 0) return 0;
  return dsa::attn_workspace_bytes(s, H, d_qk, d_v, k, dtype == DSA_BF16);
}

dsa_status_t dsa_sparse_mla_attn(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk, int32_t d_v,
                                 dsa_dtype_t dtype, const void* q, const void* kv,
                                 const int32_t* indices, int32_t k, float softmax_scale,
                                 void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  st = check_attn(s, H, d_qk, d_v, dtype, q, kv, indices, k, out, lse);
  if (st != DSA_OK) return st;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f)
    return fail(DSA_ERR_SHAPE, "softmax_scale must be positive and finite (got %g)", softmax_scale);
  const size_t need = dsa::attn_workspace_bytes(s, H, d_qk, d_v, k, dtype == DSA_BF16);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "attention workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return run_attn(s, H, d_qk, d_v, dtype, q, kv, indices, k, softmax_scale, out, lse, ws,
                  ws_bytes, static_cast<hipStream_t>(stream));
}

size_t dsa_forward_workspace_size(const dsa_seqs_t* seqs, const dsa_forward_args_t* args) {
  dsa::SeqInfo s;
  if (!args || check_seqs(seqs, s) != DSA_OK || s.B == 0 || args->k < 1) return 0;
  return plan_forward(s, args).total;
}

dsa_status_t dsa_forward(const dsa_seqs_t* seqs, const dsa_forward_args_t* a, void* ws,
                         size_t ws_bytes, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (!a) return fail(DSA_ERR_NULL, "args is NULL");
  if (s.B == 0) return ok();
  st = check_forward(s, a);
  if (st != DSA_OK) return st;
  const ForwardPlan p = plan_forward(s, a);
  const int64_t ld = a->scores_out ? a->ld_scores_out : p.ld;
  if (p.total > 0 && (!ws || ws_bytes < p.total))
    return fail(DSA_ERR_WORKSPACE, "forward workspace needs %zu bytes, got %zu", p.total, ws_bytes);
  if (ws && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DSA_ERR_ALIGN, "forward workspace must be %zu-byte aligned", kAlign);
  if (s.T == 0) return ok();
  char* base = static_cast<char*>(ws);
  // (without the indexer, the top-k kernels never read the scores: every row has n <= k)
  float* scores = a->scores_out ? a->scores_out
                                : (p.scores_bytes ? reinterpret_cast<float*>(base + p.scores_off) : nullptr);
  int32_t* idx = a->indices_out ? a->indices_out
                                : (p.idx_bytes ? reinterpret_cast<int32_t*>(base + p.idx_off) : nullptr);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (p.run_indexer) {
    st = run_indexer(s, a->H_I, a->d_I, a->qk_dtype, a->q_idx, a->q_idx_scale, a->k_idx,
                     a->k_idx_scale, a->w, scores, ld, p.index_bytes ? base + p.index_off : nullptr, hs);
    if (st != DSA_OK) return st;
  }
  if (p.run_topk) {
    st = hip_status(dsa::launch_topk(s, scores, ld, a->k, idx, p.topk_bytes ? base + p.topk_off : nullptr,
                                     p.topk_bytes, hs),
                    "top-k launch");
    if (st != DSA_OK) return st;
  }
  return run_attn(s, a->H, a->d_qk, a->d_v, a->dtype, a->q, a->kv, p.implicit_idx ? nullptr : idx,
                  a->k, a->softmax_scale, a->out, a->lse, p.attn_bytes ? base + p.attn_off : nullptr,
                  p.attn_bytes, hs, p.run_topk);
}

dsa_status_t dsa_forward_noalloc(const dsa_seqs_t* seqs, const dsa_forward_args_t* args, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (!args) return fail(DSA_ERR_NULL, "args is NULL");
  if (s.B == 0) return ok();
  st = check_forward(s, args);
  if (st != DSA_OK) return st;
  const size_t need = plan_forward(s, args).total;
  if (need > DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE, "dsa_forward_noalloc: this batch needs %zu bytes of workspace, more than "
                "the %llu-byte scratch (use dsa_forward with a caller workspace)", need,
                (unsigned long long)DSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != DSA_OK) return st;
  }
  return dsa_forward(seqs, args, ws, need, stream);
}

dsa_status_t dsa_indexer_alignment(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk, dsa_dtype_t dtype,
                                   const void* q, const void* kv, const int32_t* indices, int32_t k,
                                   float softmax_scale, const float* lse, const float* scores,
                                   int64_t ld_scores, float* target, float* kl, void* stream) {
  dsa::SeqInfo s;
  dsa_status_t st = check_seqs(seqs, s);
  if (st != DSA_OK) return st;
  if (s.B == 0) return ok();
  if (dtype != DSA_BF16 && dtype != DSA_F32)
    return fail(DSA_ERR_DTYPE, "alignment inputs must be DSA_BF16 (DSA_F32 is not implemented)");
  if (dtype != DSA_BF16 || H != 128 || d_qk != 576)
    return fail(DSA_ERR_UNSUPPORTED, "the alignment target needs bf16 with (H, d_qk) = (128, 576)");
  if (k < 1 || k > 16384) return fail(DSA_ERR_UNSUPPORTED, "k = %d outside 1..16384", k);
  if (ld_scores < s.max_n || ld_scores % 4 != 0)
    return fail(DSA_ERR_SHAPE, "ld_scores = %lld must be >= max_seqlen_k (%d) and a multiple of 4",
                (long long)ld_scores, s.max_n);
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f)
    return fail(DSA_ERR_SHAPE, "softmax_scale must be positive and finite (got %g)", softmax_scale);
  if ((int64_t)s.max_n * d_qk * 2 > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "needs max_seqlen_k * 1152 < 2^31 (got %d keys)", s.max_n);
  if (s.T == 0) return ok();
  if (!q || !kv || !indices || !lse || !scores || !kl)
    return fail(DSA_ERR_NULL, "alignment tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(indices) || !aligned16(lse) || !aligned16(scores) ||
      !aligned16(kl) || (target && !aligned16(target)))
    return fail(DSA_ERR_ALIGN, "alignment tensors must be 16-byte aligned");
  return hip_status(dsa::launch_align_bf16(s, static_cast<const uint16_t*>(q),
                                           static_cast<const uint16_t*>(kv), indices, k, softmax_scale,
                                           lse, scores, ld_scores, target, kl,
                                           static_cast<hipStream_t>(stream)),
                    "alignment launch");
}

const char* dsa_status_string(dsa_status_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "inconsistent shape";
    case DSA_ERR_DTYPE: return "unsupported storage type for this argument";
    case DSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "configuration not implemented";
    case DSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* dsa_last_error(void) { return g_err; }

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

}  // extern "C"
