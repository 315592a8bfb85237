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
hipError_t launch_indexer_fp8_decode(const SeqInfo& s, const uint8_t* q, const uint8_t* k,
                                     const float* w, const float* kscale, float* scores,
                                     int64_t ld, hipStream_t st);
// weff = w * qscale elementwise ([T, H_I]).
hipError_t launch_indexer_scale_weights(const SeqInfo& s, int H_I, const float* w, const float* qscale,
                                        float* weff, hipStream_t st);

// ---------------------------------------------------------------- top-k
size_t topk_workspace_bytes(const SeqInfo& s, int k);
hipError_t launch_topk(const SeqInfo& s, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, size_t ws_bytes, hipStream_t st);

// ---------------------------------------------------------------- attention
size_t attn_workspace_bytes(const SeqInfo& s, int H, int d_qk, int d_v, int k, bool bf16);
hipError_t launch_attn_f32(const SeqInfo& s, int H, int d_qk, int d_v, const float* q,
                           const float* kv, const int32_t* idx, int k, float scale, float* out,
                           float* lse, hipStream_t st);
hipError_t launch_attn_bf16(const SeqInfo& s, const uint16_t* q, const uint16_t* kv,
                            const int32_t* idx, int k, float scale, uint16_t* out, float* lse,
                            void* ws, size_t ws_bytes, hipStream_t st);

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
