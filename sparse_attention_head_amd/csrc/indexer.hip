// Lightning-indexer scores on gfx950.
//
//   I[r, s] = sum_j w[r, j] * ReLU(qI[r, j] . kI[s])      for s = 0..pos(r)
//
// (page "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models" (paper digest),
//  section "Key claims": paper section 2.1, Eq. 1 -- few indexer heads, ReLU, FP8. Page "A paper
//  signed by Liang Wenfeng: The most powerful open-source Agent model of DeepSeek has made a big
//  splash" (36kr), section "02. Built on the final version of DeepSeek-V3.1, DSA makes model
//  computation smarter": index scores between a query token and the tokens before it.)
//
// FP8 path (H_I = 64, d_I = 128). The score is a dense contraction: for a block of query rows the
// products qI[r, j] . kI[s] form a GEMM of shape [rows * 64 heads, 128] x [128, keys]. d_I = 128
// is exactly one K step of v_mfma_f32_16x16x128_f8f6f4, so every 16x16 output tile costs a single
// matrix instruction; the ReLU and the weighted head sum run on the vector ALU straight out of the
// accumulator registers (2 VALU ops per (row, head, key)), so nothing but the final score leaves
// the registers.
//
// MFMA operand mapping. A 16x16x128 output tile has M = 16 (row, head) pairs and N = 16 keys.
// Lane l holds output column l%16 and rows 4*(l/16)+v, v = 0..3. The M index is laid out as
// (row-in-wave, head) so that a lane's 4 values belong to one query row: with RW rows per wave and
// HPM = 16/RW heads per row in a tile, M index i = row * HPM + head_local. For RW = 4 every lane
// owns one row and the head sum never leaves the lane; for RW = 2 / 1 the partial sums of 2 / 4
// lane groups are added with cross-lane swaps at the end of each key block.
// The K (d_I) index is split across lane groups identically for A (queries) and B (keys), so the
// contraction does not depend on the hardware's byte order within a lane.
// That is the mapping of the decode (one row per workgroup) kernel. The prefill kernel further
// down swaps the roles (keys as the A operand, 4 rows x 4 heads per tile as B), stages the keys
// in LDS for all 8 waves of a workgroup, and halves the epilogue with the split ReLU identity
// and an extra matrix tile for its linear term.
#include "dsa_internal.h"
#include "device_common.h"

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------- fp32 vector path

__global__ void __launch_bounds__(256)
indexer_f32_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                   int H_I, int d_I, const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ w, const float* __restrict__ kscale,
                   float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sm[];  // q row [H_I * d_I], then w row [H_I]
  const int r = blockIdx.x;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int s0 = blockIdx.y * 256;
  if (s0 > L.pos) return;  // uniform over the block
  float* qs = sm;
  float* ws = sm + H_I * d_I;
  for (int i = threadIdx.x; i < H_I * d_I; i += 256) qs[i] = q[(int64_t)r * H_I * d_I + i];
  for (int i = threadIdx.x; i < H_I; i += 256) ws[i] = w[(int64_t)r * H_I + i];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s > L.pos) return;
  const float* kr = k + (int64_t)(L.kofs + s) * d_I;
  float acc = 0.f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < d_I; ++d) dot = fmaf(qs[j * d_I + d], kr[d], dot);
    acc = fmaf(ws[j], fmaxf(dot, 0.f), acc);
  }
  if (kscale) acc *= kscale[L.kofs + s];   // per-key scale of the keys (positive)
  scores[(int64_t)r * ld + s] = acc;
}

hipError_t launch_indexer_f32(const SeqInfo& s, int H_I, int d_I, const float* q, const float* k,
                              const float* w, const float* kscale, float* scores, int64_t ld,
                              hipStream_t st) {
  if (s.T == 0 || s.max_n == 0) return hipSuccess;
  dim3 grid(s.T, (s.max_n + 255) / 256);
  size_t lds = (size_t)(H_I * d_I + H_I) * sizeof(float);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), lds, st, s.B, s.cu_q, s.cu_k, H_I, d_I,
                     q, k, w, kscale, scores, ld);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- scale factors
// Per-(row, head) query scales a_rj > 0 fold into the head weights: ReLU(a x) = a ReLU(x), so
// sum_j w_j ReLU(a_j q_j . k) = sum_j (w_j a_j) ReLU(q_j . k). The kernels then run on w * a.
__global__ void __launch_bounds__(256)
indexer_scale_weights_kernel(int64_t count, const float* __restrict__ w, const float* __restrict__ qs,
                             float* __restrict__ weff) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) weff[i] = w[i] * qs[i];
}

hipError_t launch_indexer_scale_weights(const SeqInfo& s, int H_I, const float* w, const float* qscale,
                                        float* weff, hipStream_t st) {
  const int64_t count = (int64_t)s.T * H_I;
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_scale_weights_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     st, count, w, qscale, weff);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- FP8 matrix path

constexpr int kHI = 64;     // indexer heads
constexpr int kDI = 128;    // indexer head dim (bytes per FP8 vector)

__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // format codes 0/0 = FP8 E4M3 for both operands; no block scaling
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Same with the B operand scaled per lane: 2^(b_scale - 127) on lane l's column (l % 16) and its
// K block (l / 16); A unscaled (127 = 1.0).
__device__ __forceinline__ v4f mfma_fp8_16x16x128_bscale(const v8i& a, const v8i& b, int b_scale) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, b_scale);
}

// ReLU on the bit pattern: a non-negative IEEE float is a non-negative int32 and a negative one
// (including -0) a negative int32, so max(bits, 0) is ReLU with one integer instruction (the
// float max would first canonicalise its operand).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Computes the scores of RW query rows (one wave) against 16 keys held in `bop`.
// Returns, per lane, the partial head sum for (row g*RW/4, key l%16) over the heads this lane
// owns; the caller completes it across lane groups when RW < 4. Matrix instructions and the
// ReLU/weight epilogue are interleaved, so only a few tiles are live at a time and the vector work
// overlaps the matrix work (two waves share each SIMD and fill each other's dependency stalls).
template <int RW>
__device__ __forceinline__ float score_block(const v8i (&a)[4 * RW], const v8i& bop,
                                             const float (&wv)[16 * RW]) {
  constexpr int NMF = 4 * RW;  // MFMAs per key block: RW rows * 64 heads / 16
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mm = 0; mm < NMF; ++mm) {
    const v4f d = mfma_fp8_16x16x128(a[mm], bop);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = fmaf(wv[4 * mm + v], relu_bits(d[v]), acc[v]);
  }
  // pipeline for the machine scheduler: matrix instructions run ahead of the epilogue, one
  // matrix instruction per 8 vector instructions
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
  for (int i = 0; i < NMF - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 19, 0);
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// ---------------------------------------------------------------------------- prefill, LDS-staged keys
// The epilogue above costs two vector instructions (max, fma) per (row, head, key), as much vector
// time as the matrix instruction that produced the 4 values takes, so it, not the matrix core,
// bounded the kernel. The prefill path halves it with the identity
//
//   sum_j w_j max(0, x_j) = 1/2 sum_j w_j |x_j|  +  1/2 sum_j w_j x_j ,
//
// whose first sum is one fma per value (|x| is a free source modifier) and whose second sum is
// linear in the key: sum_j w_j (qI_j . k) = u . k with u = sum_j w_j qI_j, one 128-long vector
// per query row. That dot product runs on the matrix core as one extra 16x16x128 tile per 16 keys:
// u is split into 4 FP8 pieces, u * 2^-e = sum_p c_p 16^-p + residual (e per row makes
// max|u * 2^-e| fall in [128, 256); each piece is the round-to-nearest-even E4M3 value of the
// previous remainder times 16), and the tile's M index is (row, piece). The remainder after 4
// pieces is at most 2^-16 |u_d| + 2^-22 * 2^e per component; integer-valued inputs split exactly.

// Round to the nearest (ties to even) value of the E4M3 grid; |r| < 448.
__device__ __forceinline__ float round_e4m3(float r) {
  uint32_t b = __float_as_uint(r);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & ~0xFFFFFu;           // 3 fraction bits, normal range
  const float sub = rintf(r * 512.f) * (1.f / 512.f);           // subnormal grid, multiples of 2^-9
  return fabsf(r) < 0x1p-6f ? sub : __uint_as_float(b);
}

// E4M3 code of a value that lies on the E4M3 grid.
__device__ __forceinline__ uint32_t encode_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const float a = fabsf(v);
  const uint32_t mag = a < 0x1p-6f ? (uint32_t)(a * 512.f)
                                   : ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
  return ((b >> 24) & 0x80u) | mag;
}

// Value of an E4M3 code: the code's low 7 bits placed at the top of an fp32 fraction give the
// value times 2^-120 for normal and subnormal codes alike.
__device__ __forceinline__ float decode_e4m3(uint32_t c) {
  return __uint_as_float(((c & 0x80u) << 24) | ((c & 0x7Fu) << 20)) * 0x1p120f;
}

constexpr int LIN_BYTES = 4 * kDI;   // pieces of one row: [4][128] codes

// One wave per row, two dims per lane: u = sum_j w_j qI_j, the row's exponent e and the 4 pieces.
// pieces [T][4][128] codes; piece_exp [T] = 126 + e, the E8M0 code of 2^(e-1) (the matrix
// instruction applies 2^(e-1) * 16^-p to piece p through its per-column scale operand).
__global__ void __launch_bounds__(256)
indexer_fp8_linear_kernel(int T, const uint8_t* __restrict__ q, const float* __restrict__ w,
                          uint8_t* __restrict__ pieces, int32_t* __restrict__ piece_exp) {
  const int r0 = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (r0 >= T) return;   // whole wave
  const int lane = threadIdx.x & 63;
  const uint8_t* qr = q + (int64_t)r0 * (kHI * kDI) + 2 * lane;
  const float* wr = w + (int64_t)r0 * kHI;
  float u0 = 0.f, u1 = 0.f;
#pragma unroll 16
  for (int j = 0; j < kHI; ++j) {
    const uint32_t c = *reinterpret_cast<const uint16_t*>(qr + j * kDI);
    const float wj = wr[j];
    u0 = fmaf(wj, decode_e4m3(c), u0);
    u1 = fmaf(wj, decode_e4m3(c >> 8), u1);
  }
  float mx = fmaxf(fabsf(u0), fabsf(u1));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  int ex = 0;
  if (mx > 0.f) {
    frexpf(mx, &ex);   // mx = f * 2^ex, f in [0.5, 1)
    // max |u| * 2^-ex in [128, 256); the floor keeps every piece scale 2^(ex-1-4p) in the E8M0
    // range (rows with max |u| < 2^-105 then split a smaller multiple of u, still exactly
    // accounted for: the remainder stays below 2^-22 * 2^ex)
    ex = max(ex - 8, -112);
  }
  float rem0 = ldexpf(u0, -ex), rem1 = ldexpf(u1, -ex);
  uint16_t* out = reinterpret_cast<uint16_t*>(pieces + (int64_t)r0 * LIN_BYTES) + lane;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float v0 = round_e4m3(rem0), v1 = round_e4m3(rem1);
    out[p * (kDI / 2)] = (uint16_t)(encode_e4m3(v0) | (encode_e4m3(v1) << 8));
    rem0 = (rem0 - v0) * 16.f;
    rem1 = (rem1 - v1) * 16.f;
  }
  if (lane == 0) piece_exp[r0] = 126 + ex;
}

// Scores of 16 keys against the wave's 4 rows. The keys are the A operand (M index = key) and the
// query tiles the B operand (N index c -> row c/4 and head 4*mm + c%4, or piece c%4 for the linear
// tile), so lane (g, c) receives keys 4g+v, v = 0..3, for one (row, head) pair per tile and needs
// one weight per tile: wt[mm] = w[row c/4, head 4mm + c%4] / 2. The 4 lanes of a quad (c%4) then
// hold partial sums of the same row; two cross-lane steps add them so that lane (g, c) ends with
// the score of row c/4 and key 4g + c%4. The linear tile's column scale lsc (E8M0) applies
// 2^(e-1) * 16^-(c%4) to the lane's piece, so its result starts the accumulation as is.
__device__ __forceinline__ float score_block_t(const v8i (&qa)[16], const v8i& ql, const v8i& key,
                                               const float (&wt)[16], int lsc, bool hi2, bool hi1) {
  const v4f dl = mfma_fp8_16x16x128_bscale(key, ql, lsc);
  float acc[4] = {dl[0], dl[1], dl[2], dl[3]};
#pragma unroll
  for (int mm = 0; mm < 16; ++mm) {
    const v4f d = mfma_fp8_16x16x128(key, qa[mm]);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = fmaf(wt[mm], fabsf(d[v]), acc[v]);
  }
  // quad reduce-scatter: lanes with c&2 keep keys 2,3 (else 0,1), then c&1 picks one of the two
  const float k0 = hi2 ? acc[2] : acc[0], k1 = hi2 ? acc[3] : acc[1];
  const float s0 = hi2 ? acc[0] : acc[2], s1 = hi2 ? acc[1] : acc[3];
  const float n0 = k0 + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0x4E, 0xF, 0xF, true));
  const float n1 = k1 + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0x4E, 0xF, 0xF, true));
  const float kk = hi1 ? n1 : n0, ss = hi1 ? n0 : n1;
  const float r = kk + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ss), 0xB1, 0xF, 0xF, true));
  // the matrix instructions run ahead of their epilogues, 4 vector instructions apart
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
#pragma unroll
  for (int i = 0; i < 14; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
  return r;
}

// A whole stage of NB key blocks as one software pipeline of NB * 17 matrix instructions: step t
// issues matrix instruction t and the 4 vector instructions that consume the result of
// instruction t - 3 (by then complete); the cross-lane reduction of a finished block is spread
// over the next three steps. The keys of block b+1 are read from LDS while block b runs.
// Steps are instantiated at compile time (every register index is a constant) and
// sched_barrier keeps them in order.
struct PipeState {
  const uint8_t* buf;   // stage buffer + this lane's key row
  int kb0, kb1;         // this lane's two 16-byte chunks within a key row
  const v8i* qa;        // [16] head tiles
  v8i ql;               // linear tile
  const float* wt;      // [16] halved weights
  int lsc;              // E8M0 column scale of the linear tile
  bool hi2, hi1;
  float* sp;            // this lane's first score of the stage
  v8i key[2];
  v4f d[4];
  float acc[4], red[4], n0, n1, kk, ss;
};

template <int NB, int T>
__device__ __forceinline__ void pipe_step(PipeState& P) {
  constexpr int NM = 17, LAG = 3, TOT = NB * NM;
  if constexpr (T < TOT) {
    constexpr int blk = T / NM, j = T % NM;
    if constexpr (j == 1 && blk + 1 < NB) {
      const uint8_t* rowp = P.buf + (blk + 1) * 16 * kDI;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp + P.kb0);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + P.kb1);
      P.key[(blk + 1) & 1] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if constexpr (j == 0)
      P.d[T % 4] = mfma_fp8_16x16x128_bscale(P.key[blk & 1], P.ql, P.lsc);
    else
      P.d[T % 4] = mfma_fp8_16x16x128(P.key[blk & 1], P.qa[j - 1]);
  }
  constexpr int e = T - LAG;
  if constexpr (e >= 0 && e < TOT) {
    constexpr int j = e % NM;
    const v4f de = P.d[e % 4];
    if constexpr (j == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) P.acc[v] = de[v];
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) P.acc[v] = fmaf(P.wt[j - 1], fabsf(de[v]), P.acc[v]);
    }
    if constexpr (j == NM - 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) P.red[v] = P.acc[v];
    }
  }
  // reduction of block b: its last epilogue ran at step b*NM + NM-1 + LAG; r = 1..3 steps later
  constexpr int f = T - LAG - (NM - 1);
  if constexpr (f >= 1 && (f - 1) % NM == 0 && (f - 1) / NM < NB) {
    const float k0 = P.hi2 ? P.red[2] : P.red[0], k1 = P.hi2 ? P.red[3] : P.red[1];
    const float s0 = P.hi2 ? P.red[0] : P.red[2], s1 = P.hi2 ? P.red[1] : P.red[3];
    P.n0 = k0 + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0x4E, 0xF, 0xF, true));
    P.n1 = k1 + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0x4E, 0xF, 0xF, true));
  }
  if constexpr (f >= 2 && (f - 2) % NM == 0 && (f - 2) / NM < NB) {
    P.kk = P.hi1 ? P.n1 : P.n0;
    P.ss = P.hi1 ? P.n0 : P.n1;
  }
  if constexpr (f >= 3 && (f - 3) % NM == 0 && (f - 3) / NM < NB) {
    constexpr int blk = (f - 3) / NM;
    P.sp[blk * 16] = P.kk + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(P.ss), 0xB1, 0xF, 0xF, true));
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (T + 1 < TOT + LAG + 3) pipe_step<NB, T + 1>(P);
}

template <int NB>
__device__ __forceinline__ void stage_pipeline(const uint8_t* __restrict__ buf, int kb0, int kb1,
                                               const v8i (&qa)[16], const v8i& ql,
                                               const float (&wt)[16], int lsc, bool hi2, bool hi1,
                                               float* __restrict__ sp) {
  PipeState P;
  P.buf = buf;
  P.kb0 = kb0;
  P.kb1 = kb1;
  P.qa = qa;
  P.ql = ql;
  P.wt = wt;
  P.lsc = lsc;
  P.hi2 = hi2;
  P.hi1 = hi1;
  P.sp = sp;
  {
    const v4i lo = *reinterpret_cast<const v4i*>(buf + kb0);
    const v4i hi = *reinterpret_cast<const v4i*>(buf + kb1);
    P.key[0] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  pipe_step<NB, 0>(P);
}

// Workgroup = 8 waves x 4 rows = 32 query rows of one sequence against a chunk of keys. The keys
// stream through a ring of LDS stages (256 keys = 32 KB each) filled by DMA (global_load_lds); all
// waves share them. Inside a stage, key s occupies 128 bytes whose 16-byte chunk c sits at
// position c ^ key_swz(s % 16). A read of 16 consecutive keys for the A operand (lane l: key
// l%16, one chunk per lane) then touches distinct banks both within each group of 8 lanes (32
// four-byte banks cover one key row) and within each group of 16 lanes (64 banks cover two rows).
__device__ __forceinline__ int key_swz(int s16) { return ((s16 >> 1) ^ ((s16 & 1) << 2)) & 7; }

constexpr int PF_W = 8;                 // waves per workgroup
constexpr int PF_RW = 4;                // rows per wave
constexpr int PF_ROWS = PF_W * PF_RW;   // 32
constexpr int PF_SK = 256;              // keys per stage
constexpr int PF_NR = 3;                // stages in the ring
constexpr int PF_KC_MAX = 16384;        // keys per workgroup (chunk) at most
constexpr int PF_STW = PF_SK + 16;      // words per staged score row

// KS: every score is multiplied by the per-key scale kscale[key row] (positive), as a stage's
// staged rows leave (each lane's four keys share one 16-byte load of scales, requested before the
// stage's pipeline).
template <bool KS>
__global__ void __launch_bounds__(PF_W * 64, 1)
indexer_fp8_prefill_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                           const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                           const float* __restrict__ w, const uint8_t* __restrict__ lin,
                           const int32_t* __restrict__ piece_exp, const float* __restrict__ kscale,
                           float* __restrict__ scores, int64_t ld, int KC) {
  __shared__ __attribute__((aligned(1024))) uint8_t kst[PF_NR][PF_SK * kDI];
  // each wave's 4 rows x 256 scores of a whole stage collect here (rows padded to PF_STW words:
  // the pipeline's writes and the row reads are free of bank conflicts) and leave as four 1 KB row
  // stores, so that every 128-byte line of a score row is written whole at once
  __shared__ __attribute__((aligned(16))) float stw[PF_W * PF_RW * PF_STW];
  constexpr int HPM = 4, NMF = 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, chunk = blockIdx.y, i_base = blockIdx.x * PF_ROWS;
  const int q0 = cu_q[b], m = cu_q[b + 1] - q0;
  const int k0 = cu_k[b], n = cu_k[b + 1] - k0;
  if (i_base >= m) return;
  const int tile_last = min(m, i_base + PF_ROWS) - 1;
  const int kbeg = chunk * KC;
  if (kbeg > n - m + tile_last) return;                     // uniform over the workgroup
  const int kend = min(kbeg + KC, n - m + tile_last + 1);   // workgroup's key range end
  const int nst = (kend - kbeg + PF_SK - 1) / PF_SK;

  // this wave's rows (may be past m in the tile tail: computed on clamped rows, never stored)
  const int wrow0 = i_base + wave * PF_RW;
  const int wrow_last = min(m - 1, wrow0 + PF_RW - 1);
  const int wkend = wrow0 < m ? min(kend, n - m + wrow_last + 1) : kbeg;
  const bool all_rows = wrow0 + PF_RW <= m;

  // DMA of stage st: 32 instructions of 1 KB (8 keys each), 4 per wave; lane l of instruction i
  // covers key (i*8 + l/8) of the stage, whose 16 mod 16 is 8*(i%2) + l/8, and writes physical
  // chunk l%8, i.e. logical chunk (l%8) ^ key_swz(key % 16).
  const int dch0 = ((lane & 7) ^ key_swz(lane >> 3)) * 16;
  const int dch1 = ((lane & 7) ^ key_swz(8 | (lane >> 3))) * 16;
  auto issue = [&](int st) {
    uint8_t* dst = kst[st % PF_NR];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int inst = wave * 4 + i;
      const int key = kbeg + st * PF_SK + inst * 8 + (lane >> 3);
      const uint8_t* src = k + (int64_t)(k0 + min(key, n - 1)) * kDI + ((i & 1) ? dch1 : dch0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(dst + inst * 1024),
                                       16, 0, 0);
    }
  };
#pragma unroll
  for (int st = 0; st < PF_NR - 1; ++st)
    if (st < nst) issue(st);

  // query operands: head tiles (lane c -> row c/4, head 4*mm + c%4) and the linear tile (lane c ->
  // row c/4, piece c%4), K bytes 32g..32g+31; 136 registers, all architectural (the kernel uses no
  // accumulation registers, so two waves per SIMD get 256 each).
  v8i a[NMF], al;
  {
    const int ar = min(wrow0 + c / HPM, m - 1);
    const uint8_t* qrow = q + (int64_t)(q0 + ar) * (kHI * kDI) + (c % HPM) * kDI + g * 32;
#pragma unroll
    for (int mm = 0; mm < NMF; ++mm) a[mm] = *reinterpret_cast<const v8i*>(qrow + mm * HPM * kDI);
    al = *reinterpret_cast<const v8i*>(lin + (int64_t)(q0 + ar) * LIN_BYTES + (c % 4) * kDI + g * 32);
  }
  // lane (g, c) finishes row c/4 of the wave at key 4g + c%4 of each block
  const int my_i = wrow0 + (c >> 2);
  const int my_r = q0 + min(my_i, m - 1);
  float wt[16];
  {
    const float* wr = w + (int64_t)my_r * kHI + (c & 3);
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) wt[mm] = 0.5f * wr[4 * mm];
  }
  const int lsc = piece_exp[my_r] - 4 * (c & 3);
  const bool hi2 = (c & 2) != 0, hi1 = (c & 1) != 0;
  const bool row_ok = my_i < m;
  const int my_pos = n - m + my_i;
  const int kofs = 4 * g + (c & 3);   // this lane's key within a 16-key block
  float* srow = scores + (int64_t)my_r * ld;

  // B operand of 16 keys starting at stage-local key kl: lane's key kl + c, chunks 2g, 2g+1
  const int bx0 = ((2 * g) ^ key_swz(c)) * 16, bx1 = ((2 * g + 1) ^ key_swz(c)) * 16;
  auto load_b = [&](const uint8_t* buf, int kl) -> v8i {
    const uint8_t* rowp = buf + (kl + c) * kDI;
    const v4i lo = *reinterpret_cast<const v4i*>(rowp + bx0);
    const v4i hi = *reinterpret_cast<const v4i*>(rowp + bx1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Vector memory operations complete in issue order, so the wait for stage st's DMA may leave
  // the operations issued after it in flight: a whole stage's 4 row stores per wave (and, in the
  // scaled kernel, its scale load, issued before the DMA of stage st+2), the next stage's DMA (4),
  // the stores of the stage after. `fast1`/`fast2`: stage st-1 / st-2 ran the whole-stage path,
  // whose operations are certain (other stages count as 0).
  float* const stw_wave = stw + wave * PF_RW * PF_STW;
  bool fast1 = false, fast2 = false;
  for (int st = 0; st < nst; ++st) {
    const int after = (st == 0) ? 0 : PF_RW * fast2 + (PF_RW + (KS ? 1 : 0)) * fast1 + 4 * (st + 1 < nst);
    switch (after) {
      case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
      case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
      case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
      case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
    // stage st landed in every wave's part; every wave is done with the buffer the next DMA
    // refills (its reads were consumed by its matrix instructions)
    __builtin_amdgcn_s_barrier();
    const int sbase = kbeg + st * PF_SK;
    const bool fast = all_rows && sbase + PF_SK <= wkend;
    // the scales of this lane's four keys of the stage (a whole stage lies inside the row)
    float4 sc4 = make_float4(1.f, 1.f, 1.f, 1.f);
    if (KS && fast) sc4 = *reinterpret_cast<const float4*>(kscale + k0 + sbase + 4 * lane);
    if (st + PF_NR - 1 < nst) issue(st + PF_NR - 1);
    const uint8_t* buf = kst[st % PF_NR];
    fast2 = fast1;
    fast1 = fast;
    if (fast) {
      // whole stage for 4 valid rows: every score lands below wkend <= n <= ld (keys past a row's
      // own position fall in the part of the row the interface leaves unspecified)
      stage_pipeline<PF_SK / 16>(buf + c * kDI, bx0, bx1, a, al, wt, lsc, hi2, hi1,
                                 stw_wave + (c >> 2) * PF_STW + kofs);
      // (one wave writes and reads its own rows: its LDS operations complete in order)
#pragma unroll
      for (int rr = 0; rr < PF_RW; ++rr) {
        float4 v = *reinterpret_cast<const float4*>(stw_wave + rr * PF_STW + 4 * lane);
        if constexpr (KS) v = make_float4(v.x * sc4.x, v.y * sc4.y, v.z * sc4.z, v.w * sc4.w);
        *reinterpret_cast<float4*>(scores + (int64_t)(q0 + wrow0 + rr) * ld + sbase + 4 * lane) = v;
      }
    } else {
      const int nblk = min(PF_SK, wkend - sbase) > 0 ? (min(PF_SK, wkend - sbase) + 15) / 16 : 0;
      for (int blk = 0; blk < nblk; ++blk) {
        float acc = score_block_t(a, al, load_b(buf, blk * 16), wt, lsc, hi2, hi1);
        asm volatile("" ::"v"(acc));
        const int s = sbase + blk * 16 + kofs;
        if (KS) acc *= kscale[k0 + min(s, n - 1)];
        if (row_ok && s <= my_pos && s < wkend) srow[s] = acc;
      }
    }
  }
}

size_t indexer_workspace_bytes(const SeqInfo& s, bool fp8) {
  if (!fp8 || s.T == 0) return 0;
  return (size_t)s.T * LIN_BYTES + ((size_t)s.T * sizeof(float) + 255) / 256 * 256;
}

// Workgroups of a launch with key chunks of kc that have keys to score: the tile of rows i0 ..
// i0 + PF_ROWS - 1 of sequence b reaches position n_b - m_b + (its last row), so chunks 0 .. that
// position / kc are scored and the rest of the grid column leaves at once (in a causal prefill
// about half of the tile x chunk grid).
static int64_t live_workgroups(const SeqInfo& s, int kc) {
  int64_t total = 0;
  for (int b = 0; b < s.B; ++b) {
    const int m = s.cu_q_host[b + 1] - s.cu_q_host[b], n = s.cu_k_host[b + 1] - s.cu_k_host[b];
    for (int i0 = 0; i0 < m; i0 += PF_ROWS) total += (n - m + min(m, i0 + PF_ROWS) - 1) / kc + 1;
  }
  return total;
}

// Key-chunk length: long enough to amortise loading the query tile (each chunk reads it again:
// 16384-key chunks halve the query re-reads of 8192-key ones at the 128K chunk), short enough to
// give several live workgroups per compute unit (counted over the causal part of the grid only:
// the 8K prefill then takes 1024-key chunks, 1152 live workgroups, instead of 2048-key ones, 640).
static int pick_chunk(const SeqInfo& s, int cus, int align, int kc_max) {
  int kc = kc_max;
  while (kc > 512 && live_workgroups(s, kc) < 4LL * cus) kc >>= 1;
  return (kc / align) * align;
}

hipError_t launch_indexer_fp8_prefill(const SeqInfo& s, const uint8_t* q, const uint8_t* k,
                                      const float* w, const float* kscale, float* scores,
                                      int64_t ld, void* ws, hipStream_t st) {
  if (s.T == 0 || s.max_n == 0) return hipSuccess;
  uint8_t* pieces = static_cast<uint8_t*>(ws);
  int32_t* piece_exp = reinterpret_cast<int32_t*>(pieces + (size_t)s.T * LIN_BYTES);
  hipLaunchKernelGGL(indexer_fp8_linear_kernel, dim3((s.T + 3) / 4), dim3(256), 0, st, s.T, q, w,
                     pieces, piece_exp);
  const int tiles = (s.max_m + PF_ROWS - 1) / PF_ROWS;
  const int kc = pick_chunk(s, kTargetCUs, PF_SK, PF_KC_MAX);
  dim3 grid(tiles, (s.max_n + kc - 1) / kc, s.B);
  if (kscale)
    hipLaunchKernelGGL(indexer_fp8_prefill_kernel<true>, grid, dim3(PF_W * 64), 0, st, s.B, s.cu_q,
                       s.cu_k, q, k, w, pieces, piece_exp, kscale, scores, ld, kc);
  else
    hipLaunchKernelGGL(indexer_fp8_prefill_kernel<false>, grid, dim3(PF_W * 64), 0, st, s.B, s.cu_q,
                       s.cu_k, q, k, w, pieces, piece_exp, kscale, scores, ld, kc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- decode
// One query row per sequence. Workgroup = 4 waves, one row, one chunk of kDecodeChunk keys; wave w
// scores the chunk's 16-key blocks w, w + 4, ... The keys reach LDS by DMA, each instruction
// copying 8 whole 128-byte key rows (1 KB contiguous in memory), into a ring of DK_NR block
// slots per wave (no cross-wave synchronisation: a wave waits for its own DMAs only); the block's
// operand is read back in the prefill kernel's swizzled layout, free of bank conflicts. The
// queries are the A operand (M index c -> head 16 mm + c), four matrix instructions per block, the
// ReLU and weighted head sum on the vector unit (score_block). The scores collect in LDS and go
// out at the end as whole lines. With a candidate buffer (fused top-k), the workgroup then keeps
// every key at or above a cut chosen from a histogram of the chunk's scores so that at least
// decode_chunk_target(n, k) keys pass, and records the count, the cut and flags.
constexpr int DK_W = 4;                 // waves per workgroup
constexpr int DK_BLK = 16 * kDI;        // bytes of a 16-key block
constexpr int DK_THREADS = DK_W * 64;
// Block slots per wave: 4 for the scores alone (three workgroups per compute unit), 3 with the
// fused top-k (four per compute unit, so that the other workgroups' key streams cover the chunk
// cut's barriers). Measured against 6 slots and two workgroups per compute unit: the ragged batch's
// indexer 198 -> 192 us, the fused indexer -> top-k 80 -> 71 us (32K decode batch) and
// 261 -> 223 us (ragged batch).
template <bool FUSED>
constexpr int dk_slots() { return FUSED ? 3 : 4; }

// s_waitcnt vmcnt(n), n rounded down to an even value <= 12 (two operations per block slot)
__device__ __forceinline__ void vm_wait_even(int n) {
  static_assert(dk_slots<false>() <= 6 && dk_slots<true>() <= 6, "vm_wait_even covers up to 12 outstanding operations");
  switch (n) {
    case 12: case 13: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 10: case 11: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 8: case 9: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 6: case 7: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 4: case 5: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 2: case 3: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

template <bool FUSED, bool KS>
__global__ void __launch_bounds__(DK_THREADS, FUSED ? 4 : 3)
indexer_fp8_decode_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                          const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                          const float* __restrict__ w, const float* __restrict__ kscale,
                          float* __restrict__ scores, int64_t ld, DecodeCand cand) {
  constexpr int DK_NR = dk_slots<FUSED>();
  __shared__ __attribute__((aligned(1024))) uint8_t ring[DK_W][DK_NR][DK_BLK];
  __shared__ __attribute__((aligned(1024))) uint8_t qt[kHI * kDI + 1024];   // query tile, then weights
  __shared__ __attribute__((aligned(16))) float sc[kDecodeChunk];
  // the fused cut's histogram (2048 words) takes the query tile's place: the tile has been read
  // into registers before the first key block, long before the cut
  uint32_t* const hist = reinterpret_cast<uint32_t*>(qt);
  static_assert(sizeof(qt) >= 2048 * sizeof(uint32_t), "the histogram fits the query tile");
  __shared__ uint32_t s_digit, s_above, s_cnt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.y, chunk = blockIdx.x;
  // all four offsets are requested before either test, so that a workgroup past its row's end
  // (half of a ragged batch's grid) leaves after one memory round trip
  const int r = cu_q[b], r1 = cu_q[b + 1];
  const int k0 = cu_k[b], n = cu_k[b + 1] - k0;    // the row sits at position n - 1
  const int kbeg = chunk * kDecodeChunk;
  if (r1 == r || kbeg >= n) return;                // no query row, or a chunk past the row's end
  const int cnt = min(kDecodeChunk, n - kbeg);
  const int nblk = (cnt + 15) >> 4;
  const int nmine = nblk > wave ? (nblk - wave + DK_W - 1) / DK_W : 0;

  // the sequence's keys as a buffer (n * 128 < 2^31 is checked on the host). DMA of the wave's
  // block jb (chunk block wave + 4 jb) into slot jb % DK_NR: instruction i copies keys 8i .. 8i + 7
  // of the block; lane l reads key 8i + l/8 (clamped to the last key; such rows are never stored),
  // logical 16-byte chunk (l % 8) ^ key_swz(8i + l/8), which lands at physical chunk l % 8.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(k + (int64_t)k0 * kDI), (short)0, n * kDI, 0x00020000);
  const uint32_t ring_base = lds_addr(&ring[wave][0][0]);
  const int ch0 = ((lane & 7) ^ key_swz(lane >> 3)) * 16, ch1 = ((lane & 7) ^ key_swz(8 | (lane >> 3))) * 16;
  auto dma = [&](int jb) {
    const int key0 = kbeg + (wave + DK_W * jb) * 16 + (lane >> 3);
    const int slot = (jb % DK_NR) * DK_BLK;
    lds_dma16(rs, ring_base, slot, min(key0, n - 1) * kDI + ch0, 0);
    lds_dma16(rs, ring_base, slot + 1024, min(key0 + 8, n - 1) * kDI + ch1, 0);
  };
  // The row's query tile (8 KB) and head weights (256 B) come in by DMA too, before the keys:
  // every vector memory operation of the main loop is then one of ours, counted exactly (a plain
  // load would make the compiler wait for all outstanding ones inside the loop).
  {
    const __amdgpu_buffer_rsrc_t qs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(q + (int64_t)r * (kHI * kDI)), (short)0, kHI * kDI, 0x00020000);
    const uint32_t qt_base = lds_addr(qt);
    lds_dma16(qs, qt_base, (2 * wave) * 1024, lane * 16, (2 * wave) * 1024);
    lds_dma16(qs, qt_base, (2 * wave + 1) * 1024, lane * 16, (2 * wave + 1) * 1024);
    if (wave == 0) {   // lanes past the 256 weight bytes read zeros (outside the buffer)
      const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(w + (int64_t)r * kHI), (short)0, kHI * 4, 0x00020000);
      lds_dma16(wsr, qt_base, kHI * kDI, lane * 16, 0);
    }
  }
#pragma unroll
  for (int jb = 0; jb < DK_NR; ++jb)
    if (jb < nmine) dma(jb);
  // the query tile and weights have landed once only the key DMAs issued after them are in flight
  vm_wait_even(2 * min(DK_NR, nmine));
  __syncthreads();

  // A operand: M index c -> head 16 mm + c, K bytes of lane group g; weights of the lane's
  // outputs (D row 4g + v -> head 16 mm + 4g + v)
  v8i a[4];
  {
    const uint8_t* qrow = qt + c * kDI + g * 32;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const v4i lo = *reinterpret_cast<const v4i*>(qrow + mm * 16 * kDI);
      const v4i hi = *reinterpret_cast<const v4i*>(qrow + mm * 16 * kDI + 16);
      a[mm] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) asm volatile("" : "+a"(a[mm]));
  }
  float wv[16];
  {
    const float* wr = reinterpret_cast<const float*>(qt + kHI * kDI);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int v = 0; v < 4; ++v) wv[4 * mm + v] = wr[mm * 16 + 4 * g + v];
  }
  // B operand of a block: lane (g, c) takes logical chunks 2g, 2g + 1 of key c
  const int bx0 = ((2 * g) ^ key_swz(c)) * 16, bx1 = ((2 * g + 1) ^ key_swz(c)) * 16;
  for (int jb = 0; jb < nmine; ++jb) {
    // block jb has landed once at most the DMAs of the (up to DK_NR - 1) later blocks are in flight
    vm_wait_even(2 * min(DK_NR - 1, nmine - 1 - jb));
    const uint8_t* rowp = &ring[wave][jb % DK_NR][0] + c * kDI;
    const v4i lo = *reinterpret_cast<const v4i*>(rowp + bx0);
    const v4i hi = *reinterpret_cast<const v4i*>(rowp + bx1);
    float acc = score_block<1>(a, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), wv);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (g == 0) sc[(wave + DK_W * jb) * 16 + c] = acc;
    if (jb + DK_NR < nmine) {   // refill this slot: its reads have completed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma(jb + DK_NR);
    }
  }
  __syncthreads();   // the chunk's scores are in LDS

  // scores out as whole lines (entries past the row's end land in the part of the row that is
  // left unspecified: ld >= round_up(n, 4)); per-key scales applied here
  float* srow = scores + (int64_t)r * ld + kbeg;
  for (int i = 4 * tid; i < cnt; i += 4 * DK_THREADS) {
    float4 v = *reinterpret_cast<const float4*>(&sc[i]);
    if (KS) {
      const float* ks = kscale + k0 + kbeg + i;
      v.x *= ks[0];
      if (i + 1 < cnt) v.y *= ks[1];
      if (i + 2 < cnt) v.z *= ks[2];
      if (i + 3 < cnt) v.w *= ks[3];
      *reinterpret_cast<float4*>(&sc[i]) = v;
    }
    *reinterpret_cast<float4*>(srow + i) = v;
  }
  if constexpr (FUSED) {
    if (n <= cand.k) return;   // uniform: every candidate of the row is selected
    const int target = decode_chunk_target(n, cand.k);
    const int cap = decode_chunk_capacity(n, cand.k);
    const int64_t cell = (int64_t)r * cand.nch + chunk;
    uint32_t* mrow = cand.meta + cell * 4;
    uint32_t* krow = cand.key + cell * cand.stride;
    uint32_t* prow = cand.pos + cell * cand.stride;
    if (KS) __syncthreads();   // the scaled scores are in LDS
    if (cnt <= target) {       // uniform: keep every key
      for (int i = tid; i < cnt; i += DK_THREADS) {
        krow[i] = float_to_ordered(sc[i]);
        prow[i] = (uint32_t)(kbeg + i);
      }
      if (tid == 0) {
        mrow[0] = (uint32_t)cnt;
        mrow[1] = 0u;
        mrow[2] = 1u;
      }
      return;
    }
    // the bin of the top 11 key bits holding the target-th largest key; if that keeps more than
    // 16 keys beyond the target, the bin of the next 11 bits inside it (keeping the merge's list
    // short); more than `cap` even then (ties) marks the chunk as overflowing
    for (int i = tid; i < 2048; i += DK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += DK_THREADS) atomicAdd(&hist[float_to_ordered(sc[i]) >> 21], 1u);
    __syncthreads();
    select_bin(hist, 2048, (uint32_t)target, &s_digit, &s_above);
    const uint32_t d1 = s_digit, above1 = s_above;
    uint32_t cut = d1 << 21, keep = above1 + hist[d1];
    if (keep > (uint32_t)target + 16u) {   // uniform
      __syncthreads();            // every thread has read hist[d1]
      for (int i = tid; i < 2048; i += DK_THREADS) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < cnt; i += DK_THREADS) {
        const uint32_t u = float_to_ordered(sc[i]);
        if ((u >> 21) == d1) atomicAdd(&hist[(u >> 10) & 2047u], 1u);
      }
      __syncthreads();
      select_bin(hist, 2048, (uint32_t)target - above1, &s_digit, &s_above);
      cut |= s_digit << 10;
      keep = above1 + s_above + hist[s_digit];
    }
    const bool over = keep > (uint32_t)cap;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    if (!over) {
      for (int i = tid; i < cnt; i += DK_THREADS) {
        const uint32_t u = float_to_ordered(sc[i]);
        if (u >= cut) {
          const uint32_t at = atomicAdd(&s_cnt, 1u);   // < keep <= cap <= stride
          krow[at] = u;
          prow[at] = (uint32_t)(kbeg + i);
        }
      }
    }
    if (tid == 0) {
      mrow[0] = over ? 0u : keep;
      mrow[1] = cut;
      mrow[2] = over ? 2u : 0u;
    }
  }
}

bool decode_fused_topk_ok(const SeqInfo& s, int k) {
  return s.max_m == 1 && k <= 2048 && s.max_n <= 131072;
}

// Candidate slots per chunk: the capacity of the row with the fewest keys among those with more
// than k (the capacity shrinks as rows grow).
static int decode_cand_stride(const SeqInfo& s, int k) {
  int nmin = 0;
  for (int b = 0; b < s.B; ++b) {
    const int m = s.cu_q_host[b + 1] - s.cu_q_host[b], n = s.cu_k_host[b + 1] - s.cu_k_host[b];
    if (m > 0 && n > k && (nmin == 0 || n < nmin)) nmin = n;
  }
  return nmin ? decode_chunk_capacity(nmin, k) : 1;
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t decode_cand_bytes(const SeqInfo& s, int k) {
  const size_t nch = (size_t)(s.max_n + kDecodeChunk - 1) / kDecodeChunk;
  const size_t cells = (size_t)s.T * nch;
  return 2 * round256(cells * decode_cand_stride(s, k) * sizeof(uint32_t)) + round256(cells * 16);
}

DecodeCand decode_cand_layout(const SeqInfo& s, int k, void* ws) {
  DecodeCand d;
  d.nch = (s.max_n + kDecodeChunk - 1) / kDecodeChunk;
  d.stride = decode_cand_stride(s, k);
  d.k = k;
  const size_t cells = (size_t)s.T * d.nch;
  const size_t kb = round256(cells * d.stride * sizeof(uint32_t));
  char* p = static_cast<char*>(ws);
  d.key = reinterpret_cast<uint32_t*>(p);
  d.pos = reinterpret_cast<uint32_t*>(p + kb);
  d.meta = reinterpret_cast<uint32_t*>(p + 2 * kb);
  return d;
}

hipError_t launch_indexer_fp8_decode(const SeqInfo& s, const uint8_t* q, const uint8_t* k,
                                     const float* w, const float* kscale, float* scores,
                                     int64_t ld, const DecodeCand* cand, hipStream_t st) {
  if (s.T == 0 || s.max_n == 0) return hipSuccess;
  const dim3 grid((s.max_n + kDecodeChunk - 1) / kDecodeChunk, s.B), block(DK_THREADS);
  const DecodeCand cd = cand ? *cand : DecodeCand{};
  if (cand && kscale)
    hipLaunchKernelGGL((indexer_fp8_decode_kernel<true, true>), grid, block, 0, st, s.B, s.cu_q, s.cu_k, q, k,
                       w, kscale, scores, ld, cd);
  else if (cand)
    hipLaunchKernelGGL((indexer_fp8_decode_kernel<true, false>), grid, block, 0, st, s.B, s.cu_q, s.cu_k, q, k,
                       w, kscale, scores, ld, cd);
  else if (kscale)
    hipLaunchKernelGGL((indexer_fp8_decode_kernel<false, true>), grid, block, 0, st, s.B, s.cu_q, s.cu_k, q,
                       k, w, kscale, scores, ld, cd);
  else
    hipLaunchKernelGGL((indexer_fp8_decode_kernel<false, false>), grid, block, 0, st, s.B, s.cu_q, s.cu_k, q,
                       k, w, kscale, scores, ld, cd);
  return hipGetLastError();
}

}  // namespace dsa
