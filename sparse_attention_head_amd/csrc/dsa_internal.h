// Internal declarations shared by the host API (dsa_api.cpp) and the kernel files.
// Not part of the public ABI: include/dsa.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Launch plan inputs derived on the host from the host copies of cu_seqlens.
struct SeqInfo {
  int32_t B;            // number of sequences
  int32_t T;            // total query rows
  int32_t Nk;           // total key rows
  int32_t max_m;        // max query rows of one sequence
  int32_t max_n;        // max keys of one sequence
  const int32_t* cu_q;  // device [B+1]
  const int32_t* cu_k;  // device [B+1]
  const int32_t* cu_q_host;
  const int32_t* cu_k_host;
};

// ---------------------------------------------------------------- indexer
// kscale: per-key scale [Nk] multiplying every score of that key, or NULL.
hipError_t launch_indexer_f32(const SeqInfo& s, int H_I, int d_I, const float* q, const float* k,
                              const float* w, const float* kscale, float* scores, int64_t ld,
                              hipStream_t st);
size_t indexer_workspace_bytes(const SeqInfo& s, bool fp8);
hipError_t launch_indexer_fp8_prefill(const SeqInfo& s, const uint8_t* q, const uint8_t* k,
                                      const float* w, const float* kscale, float* scores,
                                      int64_t ld, void* ws, hipStream_t st);
// Decode batches (every sequence has at most one query row): each workgroup scores one chunk of
// kDecodeChunk keys of one row.
constexpr int kDecodeChunk = 1024;

// Fused top-k of decode rows (the indexer keeps candidates, a merge selects; see topk.hip).
// For a row of n > k keys, each chunk keeps every key at or above a cut chosen so that at least
// decode_chunk_target(n, k) of its keys pass: the chunk's expected share mu = k * chunk / n of
// the row's top k plus six standard deviations (sqrt(mu)) and 8, at most a whole chunk. The merge
// is exact whenever no chunk holds more of the row's top k than it kept, and falls back to the
// exact selection over the score row otherwise.
__host__ __device__ inline int decode_chunk_target(int n, int k) {
  const int mu = (int)(((int64_t)k * kDecodeChunk + n - 1) / n);
  int r = 0;
  while (r * r < mu) ++r;   // ceil(sqrt(mu)); mu <= kDecodeChunk when n > k
  const int c = mu + 6 * r + 8;
  return c < kDecodeChunk ? c : kDecodeChunk;
}
// Candidate slots per chunk: the target plus 64 (keys that share the cut's bin).
__host__ __device__ inline int decode_chunk_capacity(int n, int k) {
  const int c = decode_chunk_target(n, k) + 64;
  return c < kDecodeChunk ? c : kDecodeChunk;
}

struct DecodeCand {
  uint32_t* key;    // [T][nch][stride] order-preserving score keys
  uint32_t* pos;    // [T][nch][stride] sequence-local positions
  uint32_t* meta;   // [T][nch][4]: count, cut key, flags (bit 0: every key kept; bit 1: overflow)
  int nch;          // chunks per row (ceil(max_seqlen_k / kDecodeChunk))
  int stride;       // candidate slots per chunk (capacity of the row with the fewest keys)
  int k;
};
// Layout of the candidate buffers inside a workspace of decode_cand_bytes(s, k) bytes.
size_t decode_cand_bytes(const SeqInfo& s, int k);
DecodeCand decode_cand_layout(const SeqInfo& s, int k, void* ws);
// Whether the fused decode top-k covers this batch (decode rows, k <= 2048, rows up to 131072).
bool decode_fused_topk_ok(const SeqInfo& s, int k);

// Decode indexer: scores of every row into `scores`; with cand != NULL the chunks also keep their
// top-k candidates (fused top-k).
hipError_t launch_indexer_fp8_decode(const SeqInfo& s, const uint8_t* q, const uint8_t* k,
                                     const float* w, const float* kscale, float* scores,
                                     int64_t ld, const DecodeCand* cand, hipStream_t st);
// weff = w * qscale elementwise ([T, H_I]).
hipError_t launch_indexer_scale_weights(const SeqInfo& s, int H_I, const float* w, const float* qscale,
                                        float* weff, hipStream_t st);

// ---------------------------------------------------------------- top-k
size_t topk_workspace_bytes(const SeqInfo& s, int k);
hipError_t launch_topk(const SeqInfo& s, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, size_t ws_bytes, hipStream_t st);
// Second half of the fused decode top-k: per row, the exact top k of the chunks' candidates (or
// of the score row, when the candidates cannot prove it), ascending, -1 padded.
hipError_t launch_topk_merge_decode(const SeqInfo& s, const float* scores, int64_t ld, int k,
                                    int32_t* idx, const DecodeCand& cand, hipStream_t st);

// ---------------------------------------------------------------- attention
size_t attn_workspace_bytes(const SeqInfo& s, int H, int d_qk, int d_v, int k, bool bf16);
hipError_t launch_attn_f32(const SeqInfo& s, int H, int d_qk, int d_v, const float* q,
                           const float* kv, const int32_t* idx, int k, float scale, float* out,
                           float* lse, hipStream_t st);
// prefix_rows: idx comes from this library's top-k, so a row whose causal candidates all fit in k
// holds 0..pos then -1 (the attention then stops at the row's last block).
hipError_t launch_attn_bf16(const SeqInfo& s, const uint16_t* q, const uint16_t* kv,
                            const int32_t* idx, int k, float scale, uint16_t* out, float* lse,
                            void* ws, size_t ws_bytes, bool prefix_rows, hipStream_t st);

// Indexer-alignment target p [T, k] (or NULL) and KL [T] for the bf16 (128, 576) shapes.
hipError_t launch_align_bf16(const SeqInfo& s, const uint16_t* q, const uint16_t* kv,
                             const int32_t* idx, int k, float scale, const float* lse,
                             const float* scores, int64_t ld, float* target, float* kl,
                             hipStream_t st);

// Compute units of an MI355X: the launch planning targets this many workgroups. It is a constant
// (not a device query) so that workspace sizes depend on the call's arguments only; on a device
// with fewer units the same launches simply take more waves of workgroups.
constexpr int kTargetCUs = 256;

}  // namespace dsa
