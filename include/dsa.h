/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) forward path on MI355X (gfx950).
 *
 * The operation, as the pages define it -- page "DeepSeek-V3.2: Pushing the Frontier of Open Large
 * Language Models" (paper digest), sections "Key claims" (paper section 2.1, Eq. 1-2, Fig. 2) and
 * "Method"; page "A paper signed by Liang Wenfeng: The most powerful open-source Agent model of
 * DeepSeek has made a big splash" (36kr), section "02. Built on the final version of
 * DeepSeek-V3.1, DSA makes model computation smarter":
 *
 *   1. lightning indexer: for each query token t and each key s at or before it,
 *        I[t,s] = sum_j w[t,j] * ReLU(qI[t,j] . kI[s])        (H_I indexer heads, FP8 inputs)
 *   2. fine-grained selection: keep the k keys with the largest I[t,:]
 *   3. MLA in MQA mode: every one of the H query heads of token t attends (softmax) only to the
 *      selected entries of one latent vector per key that all heads share; key = the whole
 *      latent row (d_qk dims), value = its first d_v dims.
 *
 * Conventions used by every entry point
 *   - Ragged batches. Sequence b has m_b query rows and n_b keys (m_b <= n_b). Query rows of all
 *     sequences are stacked (T = sum m_b rows), keys likewise (Nk = sum n_b rows). Query i of
 *     sequence b sits at position pos = n_b - m_b + i; its candidates are keys 0..pos of its own
 *     sequence (inclusive). A prefill is m_b = n_b, a decode step m_b = 1.
 *   - Positions in score rows and index lists are sequence-local (0..n_b-1).
 *   - Tensor pointers are device pointers to dense row-major arrays, 16-byte aligned, unless
 *     marked [host]. Shapes are given in brackets, innermost dimension last.
 *   - Storage types: DSA_FP8_E4M3 = OCP FP8 E4M3 ("e4m3fn": bias 7, no infinities, max 448)
 *     as one byte per value; DSA_BF16 = bfloat16; DSA_F32 = IEEE binary32. Inputs are taken as
 *     they are: the library never quantises and applies no scale factors.
 *   - Ownership. The caller allocates and frees every buffer, including workspaces. The
 *     library does not allocate device memory and keeps no state between calls. All work is
 *     enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns without waiting; results are valid once the stream has
 *     reached that point, and inputs must stay untouched until then.
 *   - Errors. Arguments are validated on the host before anything is enqueued; on failure the
 *     call returns a non-zero status, enqueues nothing, and dsa_last_error() describes the
 *     problem (thread-local text). A failed kernel launch returns DSA_ERR_HIP. Faults inside a
 *     kernel surface at the caller's next stream synchronisation. No C++ exception crosses
 *     this interface.
 *   - Inputs must be finite; NaN or infinite inputs give unspecified values. Every call still
 *     terminates on them, and in the attention a head whose logits are not finite only makes
 *     that head's output (and lse) non-finite.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

/* Both enums are 32-bit integers. Compiled as C++ they get int32_t as their fixed underlying
 * type, so that any int32 value a caller passes (an unknown type code, a status from a newer
 * library) is a value of the type and is rejected or reported, not undefined behaviour. */
#ifdef __cplusplus
#define DSA_ENUM_BASE : int32_t
#else
#define DSA_ENUM_BASE
#endif

typedef enum DSA_ENUM_BASE {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                                     */
  DSA_ERR_SHAPE = 2,       /* sizes inconsistent (negative, m_b > n_b, ld too small, ...)    */
  DSA_ERR_DTYPE = 3,       /* storage type not allowed for this argument                     */
  DSA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned                        */
  DSA_ERR_WORKSPACE = 5,   /* workspace pointer NULL or smaller than the *_workspace_size    */
  DSA_ERR_UNSUPPORTED = 6, /* valid request that this build does not implement              */
  DSA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed                     */
} dsa_status_t;

typedef enum DSA_ENUM_BASE { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype_t;

/* A ragged batch of sequences. The device and host arrays must hold the same values. The
 * host copies are read during the call only (validation and launch planning); the device
 * copies are read by the kernels. */
typedef struct {
  int32_t num_seqs;                    /* B >= 0; B == 0 makes every call a no-op            */
  const int32_t* cu_seqlens_q;         /* [B+1] device: 0 = c_0 <= c_1 <= ... = T            */
  const int32_t* cu_seqlens_k;         /* [B+1] device: 0 = c_0 <= c_1 <= ... = Nk           */
  const int32_t* cu_seqlens_q_host;    /* [B+1] [host] same values                            */
  const int32_t* cu_seqlens_k_host;    /* [B+1] [host] same values                            */
  int32_t max_seqlen_q;                /* max m_b (must equal the true maximum)              */
  int32_t max_seqlen_k;                /* max n_b (must equal the true maximum)              */
} dsa_seqs_t;

/* ---------------------------------------------------------------- step 1: lightning indexer
 * I[r,s] = sum_{j<H_I} w[r,j] * max(0, sum_{d<d_I} qI[r,j,d] * kI[kofs_b + s, d])
 * for every query row r (sequence b, position pos) and s = 0..pos.
 * (paper digest page, "Key claims": paper section 2.1, Eq. 1; ReLU, few heads, FP8.)
 *
 *   qk_dtype  DSA_FP8_E4M3 (H_I = 64, d_I = 128: FP8 matrix-core path; at most 65535 sequences
 *             per call) or DSA_F32 (any 1 <= H_I <= 128, 1 <= d_I <= 256, at most 65535 * 256
 *             keys per sequence: vector path). Accumulation is fp32. Outside these limits the
 *             call returns DSA_ERR_UNSUPPORTED.
 *   q_idx     [T, H_I, d_I] of qk_dtype        indexer queries
 *   k_idx     [Nk, d_I]     of qk_dtype        indexer keys, one per key token, shared by heads
 *   w         [T, H_I] fp32                    per-token head weights
 *   scores    [T, ld_scores] fp32 (output)     row r holds I[r, 0..pos]; entries beyond pos are
 *             left unspecified (they may be overwritten). ld_scores >= max_seqlen_k, and a
 *             multiple of 4.
 *   ws        device workspace of at least dsa_indexer_workspace_size(seqs, H_I, d_I, qk_dtype)
 *             bytes, 16-byte aligned (may be NULL when that size is 0); contents on entry do not
 *             matter. The FP8 path for batches with more than one query row per sequence keeps
 *             per-row data of the query side there (T * 516 bytes, rounded up).
 */
size_t dsa_indexer_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                  dsa_dtype_t qk_dtype);
dsa_status_t dsa_indexer_scores(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                dsa_dtype_t qk_dtype, const void* q_idx, const void* k_idx,
                                const float* w, float* scores, int64_t ld_scores, void* ws,
                                size_t ws_bytes, void* stream);

/* Scaled FP8 inputs. The pages give the indexer's inputs as FP8 without saying how they are
 * scaled; this call takes the common form: q_idx[r, j, :] stands for q_scale[r, j] * q_idx and
 * k_idx[s, :] for k_scale[s] * k_idx, i.e.
 *   I[r,s] = sum_j w[r,j] * ReLU((q_scale[r,j] qI[r,j]) . (k_scale[kofs_b + s] kI[kofs_b + s]))
 *          = k_scale[kofs_b + s] * sum_j (w[r,j] q_scale[r,j]) * ReLU(qI[r,j] . kI[kofs_b + s])
 * (positive homogeneity of ReLU; the kernels compute the second form).
 *   q_scale  [T, H_I] fp32 or NULL (all 1); every value positive and finite
 *   k_scale  [Nk] fp32 or NULL (all 1); every value positive and finite
 *            (other values give unspecified results; they are device data and not checked)
 *   ws       at least dsa_indexer_scaled_workspace_size(...) bytes (the unscaled call's
 *            workspace, then the scaled head weights [T, H_I] fp32), 16-byte aligned.
 * Other arguments as in dsa_indexer_scores.
 */
size_t dsa_indexer_scaled_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                         dsa_dtype_t qk_dtype);
dsa_status_t dsa_indexer_scores_scaled(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                       dsa_dtype_t qk_dtype, const void* q_idx, const float* q_scale,
                                       const void* k_idx, const float* k_scale, const float* w,
                                       float* scores, int64_t ld_scores, void* ws, size_t ws_bytes,
                                       void* stream);

/* ---------------------------------------------------------------- step 2: top-k selection
 * For each row r: the min(k, pos+1) positions s <= pos with the largest scores[r, s]
 * (36kr page, section 02: keep the entries with the top-k index scores; paper digest page,
 * "Key claims", Eq. 2). Ties prefer the lower position; +0 and -0 are equal. The positions are
 * written in ascending order to indices[r, 0..], and the rest of the row is filled with -1.
 *
 *   scores   [T, ld_scores] fp32, finite in 0..pos of every row (entries beyond are not read)
 *   k        1 <= k <= 16384
 *   indices  [T, k] int32 (output)
 *   ws       device workspace of at least dsa_topk_workspace_size(seqs, k) bytes (may be NULL
 *            when that size is 0); its contents on entry do not matter.
 */
size_t dsa_topk_workspace_size(const dsa_seqs_t* seqs, int32_t k);
dsa_status_t dsa_topk(const dsa_seqs_t* seqs, const float* scores, int64_t ld_scores, int32_t k,
                      int32_t* indices, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- steps 1 + 2 fused
 * The lightning-indexer scores and the top-k selection in one call: the same results as
 * dsa_indexer_scores followed by dsa_topk, bit for bit (paper digest page, "Key claims": paper
 * section 2.1, Eq. 1-2; 36kr page, section 02: the top-k entries by index score).
 * For decode batches (every sequence has at most one query row) with FP8 inputs (H_I = 64,
 * d_I = 128), 1 <= k <= 2048 and max_seqlen_k <= 131072, the selection is fused into the
 * indexer: each workgroup scoring a chunk of 1024 keys also keeps every key at or above a cut that
 * lets through at least the chunk's expected share of the row's top k plus six standard
 * deviations, and a merge selects the top k among the kept keys; when the kept keys cannot prove
 * the result (a chunk holding more of the top k than it kept, or too many ties), the merge selects
 * the row exactly from its scores instead. Other batches run the two steps back to back.
 *   Arguments as in dsa_indexer_scores (no scale factors) and dsa_topk; `scores` is written
 *   either way (the fused path's fallback reads it).
 *   ws  device workspace of at least dsa_indexer_topk_workspace_size(...) bytes, 256-byte
 *       aligned; contents on entry do not matter.
 */
size_t dsa_indexer_topk_workspace_size(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I,
                                       dsa_dtype_t qk_dtype, int32_t k);
dsa_status_t dsa_indexer_topk(const dsa_seqs_t* seqs, int32_t H_I, int32_t d_I, dsa_dtype_t qk_dtype,
                              const void* q_idx, const void* k_idx, const float* w, float* scores,
                              int64_t ld_scores, int32_t k, int32_t* indices, void* ws,
                              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 3: sparse MLA attention
 * For each row r (sequence b) and head h, over the selected set S = { s in indices[r, :] :
 * 0 <= s < n_b } (entries -1 or out of range are skipped; repeats count as often as listed):
 *   z_s        = softmax_scale * sum_{d<d_qk} q[r,h,d] * kv[kofs_b + s, d]
 *   out[r,h,:] = sum_s softmax(z)_s * kv[kofs_b + s, 0:d_v]
 *   lse[r,h]   = ln sum_s exp(z_s)
 * A row with an empty S gives out = 0 and lse = -inf.
 * (paper digest "Key claims", Fig. 2 and "Method": MLA in MQA mode, one latent row per key
 * shared by all query heads, attended only at the selected entries.)
 *
 *   dtype    DSA_BF16 with (H, d_qk, d_v) = (128, 576, 512) and max_seqlen_k <= 1864135 (byte
 *            offsets within one sequence's latent rows fit 31 bits; matrix-core path), or DSA_F32
 *            with 1 <= H <= 128, 1 <= d_v <= d_qk <= 1024, k <= 4096 (vector path)
 *   q        [T, H, d_qk] of dtype         queries already in the latent space
 *   kv       [Nk, d_qk] of dtype           latent cache (value = the first d_v dims)
 *   indices  [T, k] int32                  1 <= k <= 16384
 *   softmax_scale  positive and finite (DSA_ERR_SHAPE otherwise)
 *   out      [T, H, d_v] of dtype (output; bf16 rounded to nearest even)
 *   lse      [T, H] fp32 (output) or NULL
 *   ws       device workspace of at least dsa_sparse_mla_attn_workspace_size(...) bytes, 16-byte
 *            aligned (may be NULL when that size is 0); contents on entry do not matter. The bf16
 *            path splits each row's index list over several workgroups when the batch has fewer
 *            rows than the device has compute units, and keeps the per-split partial outputs
 *            (bf16) and log-sum-exps (fp32) there (splits * T * H * (2 d_v + 4) bytes). Like every
 *            *_workspace_size call, the size is a function of the arguments alone (no device
 *            query, no HIP call).
 */
size_t dsa_sparse_mla_attn_workspace_size(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk,
                                          int32_t d_v, int32_t k, dsa_dtype_t dtype);
dsa_status_t dsa_sparse_mla_attn(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk, int32_t d_v,
                                 dsa_dtype_t dtype, const void* q, const void* kv,
                                 const int32_t* indices, int32_t k, float softmax_scale,
                                 void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- fused forward (1 -> 2 -> 3)
 * Runs the three steps above on one stream for prefill and decode batches alike. Scores and
 * indices live in the workspace unless the caller asks for them through scores_out /
 * indices_out (then they are written there and also kept as the intermediate).
 * Short contexts (max_seqlen_k <= k): every row selects all its causal candidates, so the
 * indexer runs only when scores_out is given, the top-k only when indices_out is given (or for
 * the fp32 attention), and the bf16 attention walks the candidates 0..pos directly (the pages'
 * dense short-context case). The indexer arguments are still validated.
 * The call enqueues kernel launches only (no memset, copy or allocation), so it can be captured
 * into a HIP graph with the workspace and buffers it was captured with.
 */
typedef struct {
  /* indexer */
  int32_t H_I, d_I;
  dsa_dtype_t qk_dtype;
  const void* q_idx;            /* [T, H_I, d_I] */
  const void* k_idx;            /* [Nk, d_I]     */
  const float* w;               /* [T, H_I]      */
  /* selection */
  int32_t k;
  /* attention */
  int32_t H, d_qk, d_v;
  dsa_dtype_t dtype;
  const void* q;                /* [T, H, d_qk]  */
  const void* kv;               /* [Nk, d_qk]    */
  float softmax_scale;
  void* out;                    /* [T, H, d_v]   */
  float* lse;                   /* [T, H] or NULL */
  /* optional intermediates */
  float* scores_out;            /* [T, ld_scores_out] or NULL */
  int64_t ld_scores_out;
  int32_t* indices_out;         /* [T, k] or NULL */
  /* optional scales of the indexer inputs (see dsa_indexer_scores_scaled) */
  const float* q_idx_scale;     /* [T, H_I] or NULL */
  const float* k_idx_scale;     /* [Nk] or NULL */
} dsa_forward_args_t;

size_t dsa_forward_workspace_size(const dsa_seqs_t* seqs, const dsa_forward_args_t* args);
dsa_status_t dsa_forward(const dsa_seqs_t* seqs, const dsa_forward_args_t* args, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- fused forward, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it): dsa_forward with the workspace taken from a static device
 * array of DSA_NOALLOC_SCRATCH_BYTES inside the library instead of a caller buffer. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - Runs on the current device, whose own copy of the array it uses; `stream` must belong to
 *     that device. The array's address is looked up once per device (hipGetSymbolAddress), at
 *     the first call there: make that call outside a graph capture. After it, the call enqueues
 *     kernel launches only (no memset, copy or allocation) and can be captured into a HIP graph
 *     and replayed; replays read the scratch's current contents like any later call.
 *   - Batches whose dsa_forward_workspace_size exceeds DSA_NOALLOC_SCRATCH_BYTES are rejected
 *     with DSA_ERR_WORKSPACE before anything is enqueued (decode batches of up to 128 rows of
 *     128K keys fit; long prefills do not).
 *   - Every call on a device shares that device's array: calls that overlap in time on one
 *     device (different streams, or threads) race and give wrong results; serialise them. The
 *     array keeps the last call's contents; nothing in it needs to start at zero.
 * Results are identical to dsa_forward's on the same arguments.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (128ull << 20)
dsa_status_t dsa_forward_noalloc(const dsa_seqs_t* seqs, const dsa_forward_args_t* args, void* stream);

/* ---------------------------------------------------------------- indexer-alignment target
 * The training signal of the indexer (paper digest page, "Key claims", paper section 2.1.1,
 * Eq. 3-4, and "Method": a KL loss pulls the indexer's output towards the main attention's
 * distribution aggregated over the heads -- over all preceding keys in the dense warm-up, over
 * the selected entries in the sparse stage). The pages print neither equation; the reading taken:
 * for row r and its index list (entries outside 0..pos are skipped, repeats count as listed),
 *   p[r,e]  = (1/H) sum_h exp(z_{r,h,e} - lse[r,h]),  z = softmax_scale * q[r,h] . kv[kofs_b + s_e]
 *   kl[r]   = sum_e p[r,e] * (ln p[r,e] - ln softmax_e(scores[r, s_e]))       (0 ln 0 = 0)
 * i.e. each head's attention softmax over the list, averaged over the heads, against the
 * indexer's softmax over the same entries. The dense warm-up is the list 0..pos.
 *   dtype    DSA_BF16 with (H, d_qk) = (128, 576) (others: DSA_ERR_UNSUPPORTED)
 *   q, kv    as in dsa_sparse_mla_attn; indices [T, k] int32 whose entries are -1 or causal
 *            candidates (as dsa_topk produces them)
 *   lse      [T, H] fp32: the attention's log-sum-exp over the same list (dsa_sparse_mla_attn's
 *            lse output); other values give unspecified results
 *   scores   [T, ld_scores] fp32 indexer scores (entries 0..pos read)
 *   target   [T, k] fp32 (output) or NULL: p per list entry, 0 for skipped entries
 *   kl       [T] fp32 (output): 0 for a row without a valid entry
 * No workspace.
 */
dsa_status_t dsa_indexer_alignment(const dsa_seqs_t* seqs, int32_t H, int32_t d_qk, dsa_dtype_t dtype,
                                   const void* q, const void* kv, const int32_t* indices, int32_t k,
                                   float softmax_scale, const float* lse, const float* scores,
                                   int64_t ld_scores, float* target, float* kl, void* stream);

/* ---------------------------------------------------------------- misc */
const char* dsa_status_string(dsa_status_t status); /* static text, never NULL               */
const char* dsa_last_error(void);                   /* thread-local detail of the last error */
int32_t dsa_abi_version(void);                      /* DSA_ABI_VERSION of the built library  */

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
