// Sparse MLA attention in MQA mode on gfx950.
//
// For each query row and head, softmax attention over the selected latent rows only; one latent
// row per key is shared by all query heads of the token (page "DeepSeek-V3.2: Pushing the
// Frontier of Open Large Language Models" (paper digest), section "Key claims": paper section 2.1,
// Eq. 2 and Fig. 2; section "Method": MLA's MQA mode, so every selected KV entry is shared across
// the query heads). Key = the whole d_qk-dim row, value = its first d_v
// dims.
//
// BF16 matrix path (H = 128, d_qk = 576, d_v = 512), one workgroup per query row (or per run of
// whole blocks of its list, for batches with fewer rows than compute units), 4 waves, wave w owns
// heads 32w..32w+31:
//   * the selected rows are gathered 64 at a time from memory straight into LDS with
//     buffer_load_dwordx4 ... lds (no register staging), double buffered: 2 x 72 KB;
//   * S^T = K Q^T (M = 32 keys per half block, N = 32 heads, K = 576) with
//     v_mfma_f32_32x32x16_bf16; the query block of the wave stays in registers as the B operand
//     for the whole row;
//   * softmax weights in fp32 against a reference fixed for a whole pass over the row (each lane
//     owns one head), so the output accumulators are never rescaled; a half block whose weights
//     would overflow restarts the row with a larger reference;
//   * O^T += V^T P^T (M = 512 value dims, N = 32 heads, K = 32 keys); P never leaves registers:
//     the S^T accumulator layout is used directly as the B operand, and V^T is read from LDS with
//     the same permutation of the key index;
//   * the normalised rows go back to memory through LDS, one head's whole row per store; split
//     rows write bf16 partial rows and log2-sum-exps that attn_combine_kernel merges.
// LDS layout of a gathered block (16-byte slots): chunk c (dims 8c..8c+7) of key s lives in slot
//   (c / 8) * 512 + (s / 8) * 64 + (s % 8) * 8 + ((c % 8) ^ kv_swz(s % 16)).
// One DMA instruction fills 64 consecutive slots = 8 chunks of 8 keys, i.e. 8 whole 128-byte
// lines of the latent cache (fully coalesced). kv_swz keeps both read patterns free of bank
// conflicts whether the LDS serves 8 or 16 lanes of 16 bytes per cycle: the reads of one chunk of
// 16 consecutive keys (S^T) and the transposing value reads (V^T, 8 bytes per lane, 4 keys x 4
// quarter-chunks per 16 lanes). Every read splits into loop-invariant lane bits plus compile-time
// bits, so each LDS read is one of a few per-lane base registers plus an immediate offset.
#include "dsa_internal.h"
#include "device_common.h"

namespace dsa {

// ---------------------------------------------------------------------------- fp32 vector path

constexpr int AF_THREADS = 256;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < AF_THREADS / 64; ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
  return v;
}

__global__ void __launch_bounds__(AF_THREADS)
attn_f32_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int H,
                int d_qk, int d_v, const float* __restrict__ q, const float* __restrict__ kv,
                const int32_t* __restrict__ idx, int k, float scale, float* __restrict__ out,
                float* __restrict__ lse) {
  extern __shared__ float sm[];  // q vector [d_qk], logits [k], reduction [4]
  float* qs = sm;
  float* zs = sm + d_qk;
  float* red = zs + k;
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const float* qr = q + ((int64_t)r * H + h) * d_qk;
  for (int d = tid; d < d_qk; d += AF_THREADS) qs[d] = qr[d];
  __syncthreads();
  const int32_t* ir = idx + (int64_t)r * k;
  float mloc = -INFINITY;
  for (int j = tid; j < k; j += AF_THREADS) {
    const int s = ir[j];
    float z = -INFINITY;
    if (s >= 0 && s < L.n) {
      const float* c = kv + (int64_t)(L.kofs + s) * d_qk;
      float acc = 0.f;
      for (int d = 0; d < d_qk; ++d) acc = fmaf(qs[d], c[d], acc);
      z = acc * scale;
    }
    zs[j] = z;
    mloc = fmaxf(mloc, z);
  }
  const float m = block_reduce(mloc, true, red);
  float* o = out + ((int64_t)r * H + h) * d_v;
  if (m == -INFINITY) {  // no valid index
    for (int d = tid; d < d_v; d += AF_THREADS) o[d] = 0.f;
    if (lse && tid == 0) lse[(int64_t)r * H + h] = -INFINITY;
    return;
  }
  float lloc = 0.f;
  for (int j = tid; j < k; j += AF_THREADS) {
    const float p = zs[j] == -INFINITY ? 0.f : expf(zs[j] - m);
    zs[j] = p;
    lloc += p;
  }
  const float l = block_reduce(lloc, false, red);  // its barriers also publish zs
  const float inv = 1.f / l;
  for (int d = tid; d < d_v; d += AF_THREADS) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const float p = zs[j];
      if (p != 0.f) acc = fmaf(p, kv[(int64_t)(L.kofs + ir[j]) * d_qk + d], acc);
    }
    o[d] = acc * inv;
  }
  if (lse && tid == 0) lse[(int64_t)r * H + h] = m + logf(l);
}

hipError_t launch_attn_f32(const SeqInfo& s, int H, int d_qk, int d_v, const float* q,
                           const float* kv, const int32_t* idx, int k, float scale, float* out,
                           float* lse, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  size_t lds = (size_t)(d_qk + k + 8) * sizeof(float);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(s.T, H), dim3(AF_THREADS), lds, st, s.B, s.cu_q,
                     s.cu_k, H, d_qk, d_v, q, kv, idx, k, scale, out, lse);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- BF16 matrix path

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int MH = 128;            // query heads
constexpr int MDQK = 576;          // latent (key) dims
constexpr int MDV = 512;           // value dims (leading part of the latent row)
constexpr int MBLK = 64;           // keys per gathered block
constexpr int MCH = MDQK / 8;      // 16-byte chunks per latent row (72)
constexpr int MBUF = MBLK * MDQK * 2;   // bytes per LDS block buffer (73728)
constexpr int MT = MDQK / 16;      // K steps of the logits product (36)
constexpr int KRING = 4;           // LDS operand prefetch depth + 1 (logits)
constexpr int VRING = 4;           // LDS operand prefetch depth + 1 (values)

__device__ __forceinline__ v16f mfma_bf16_32x32x16(const bf16x8& a, const bf16x8& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The attention's logits product written out, so that its accumulator lives in the architectural
// registers: the output accumulators take all 256 accumulation registers, and a logits
// accumulator among them makes the compiler move one output tile in and out every half block.
// The compiler's hazard tracking does not see these instructions: a chain of them accumulates in
// place (back-to-back accumulation into the same registers needs no wait), the first one starts
// from zero (the destination is early-clobber: it must not overlap the sources), and
// logits_ready() supplies the wait states between the last one and any vector instruction that
// touches the accumulator.
__device__ __forceinline__ void logits_first(v16f& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void logits_acc(v16f& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void logits_ready(v16f& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest-even; NaN stays NaN), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Bank swizzle of the 8 chunk positions of key s (s16 = s % 16): a GF(2)-linear map whose values
// are distinct over any 8 consecutive keys and over the 8 even (odd) keys of 16, and which sends
// keys s, s+1, s+2, s+3 (s % 4 == 0) to 4 different chunk pairs, with keys s and s+2 in different
// chunk halves.
__device__ __forceinline__ int kv_swz(int s16) {
  const int b0 = (s16 >> 1) & 1, b1 = (s16 ^ (s16 >> 3)) & 1, b2 = ((s16 >> 1) ^ (s16 >> 2)) & 1;
  return b0 | (b1 << 1) | (b2 << 2);
}

// One gather instruction, untracked (UT: inline assembly, lds_dma16) or through the builtin,
// which the compiler tracks. The untracked form pays in decode, where the value product would
// otherwise wait for the next block's gather from HBM; the single-split prefill launch keeps the
// builtin.
template <bool UT>
__device__ __forceinline__ void gather16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, int lds_off, int voff,
                                         int soff) {
  if constexpr (UT) {
    lds_dma16(rsrc, lds_addr(lds), lds_off, voff, soff);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds + lds_off), 16, voff, soff, 0, 0);
  }
}

// Issue the gather of one block into `buf`. Wave w copies key groups R = 2w + u (u = 0, 1; keys
// 8R .. 8R+7) for chunk groups G = 0..8. In each instruction lane l covers key 8R + l/8 (key % 16
// = 8u + l/8) and chunk 8G + ((l % 8) ^ kv_swz(8u + l/8)), which lands in slot G*512 + R*64 + l:
// the lane-linear LDS writes of the DMA match the swizzled layout. row_u is the sequence-local
// latent row of key 8(2w + u) + l/8; `seq` addresses the sequence's rows (n * 1152 bytes).
// Buffer (not global) loads: the compiler then keeps exact LDS-read waits while they are in flight.
template <bool UT>
__device__ __forceinline__ void gather_block(uint8_t* buf, __amdgpu_buffer_rsrc_t seq, int row0,
                                             int row1, int wave, int lane, int u0 = 0, int u1 = 2) {
#pragma unroll
  for (int u = u0; u < u1; ++u) {
    const int sw = ((lane & 7) ^ kv_swz(8 * u + (lane >> 3))) * 16;
    const int voff = (u ? row1 : row0) * (MDQK * 2) + sw;
    const int R = 2 * wave + u;
#pragma unroll
    for (int G = 0; G < MCH / 8; ++G)
      gather16<UT>(seq, buf, (G * 512 + R * 64) * 16, voff, G * 128);
  }
}

// Weights are taken against a reference fixed for a whole pass over the row instead of a running
// maximum, so the output accumulators are never rescaled. A lane's weights of one half may sum to
// at most 2^60 (which keeps P, the sums and the output finite in fp32); beyond that the row is
// restarted with a larger reference.
struct SoftmaxState {
  float m;     // reference (log2 domain) used in the exponent; fixed during a pass
  float seen;  // largest half maximum recorded in this row (log2 domain): reference of a restart
  float l;     // running sum of 2^(z - m) over this lane's keys
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane i receives, as
// its element j, element (i % 4) of the 8-byte row addressed by lane 4j + i/4 of the group.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// One half block (32 keys starting at kbase inside the LDS block): logits, softmax weights,
// value accumulation. Returns true (uniform over the wave) when some head's logits exceed its
// reference by too much (see SoftmaxState); the caller then restarts the row. LDS operands are
// prefetched several MFMAs ahead. The logits loop is left to the scheduler (measured ~3 % faster
// than pinning every matrix instruction in place); in the value loop scheduling barriers keep the
// compiler from hoisting the operand reads further (which costs time and registers).
template <bool UT>
__device__ __forceinline__ bool attend_half(const uint8_t* buf, int kbase, uint32_t vmask,
                                            const bf16x8 (&qreg)[MT], v16f (&acc_o)[MDV / 32],
                                            SoftmaxState& st, float sl2, int lane,
                                            __amdgpu_buffer_rsrc_t gseq, uint8_t* gdst, int gvoff0,
                                            int gvoff1) {
  const int g = lane >> 5, c32 = lane & 31;
  // S^T = K Q^T: M = 32 keys, N = 32 heads; lane holds head c32, keys 8(i/4) + 4g + (i%4).
  // chunk c = 2t + g of key s = kbase + c32: c/8 = t/4, c%8 = 2(t%4) + g, so the slot is
  // (t/4)*512 + (s/8)*64 + (s%8)*8 + ((2(t%4) + g) ^ kv_swz(s%16)), s%16 = c32%16 (kbase is a
  // multiple of 32)
  // 4 per-lane base addresses (chunk position within the key row for t % 4); every read is one of
  // them plus an immediate offset
  const uint8_t* kb_lane = buf + (((kbase + c32) >> 3) * 64 + (c32 & 7) * 8) * 16;
  const int ksw = kv_swz(c32 & 15);
  const uint8_t* kb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) kb[q] = kb_lane + ((2 * q + g) ^ ksw) * 16;
  auto kop = [&](int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(kb[t & 3] + (t >> 2) * 8192);
  };
  v16f s;
  {
    bf16x8 ka[KRING];
#pragma unroll
    for (int t = 0; t < KRING - 1; ++t) ka[t] = kop(t);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t + KRING - 1 < MT) ka[(t + KRING - 1) % KRING] = kop(t + KRING - 1);
      if (t == 0) logits_first(s, ka[0], qreg[0]);
      else logits_acc(s, ka[t % KRING], qreg[t]);
      // gather load i = t/2 of the next block (key group 2*wave + i/9, chunk group i%9) every
      // other matrix instruction
      if ((t & 1) == 0 && gdst)
        gather16<UT>(gseq, gdst, ((t / 2) / 9) * 1024 + ((t / 2) % 9) * 8192,
                     (t / 2) / 9 ? gvoff1 : gvoff0, ((t / 2) % 9) * 128);
    }
    logits_ready(s);
  }
  // Softmax weights against the fixed reference st.m (log2 domain): p = 2^(sl2 * s - m). The
  // first half with a valid key in a pass sets the reference to its maximum; no maximum is taken
  // after that. A half whose weights in some lane sum past 2^60 (or overflow) asks for a restart
  // and records its own maximum, which the restarted pass takes as the reference.
  // Masked keys first get logit -inf (weight 0, and no part in a maximum; the scale is positive),
  // so the mask bits are only extracted for partly valid halves.
  if (vmask != 0xFFFFFFFFu) {   // uniform
    const uint32_t mlane = vmask >> (4 * g);   // bit 8(i/4) + (i%4) <-> this lane's key i
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (((mlane >> (8 * (i >> 2) + (i & 3))) & 1u) == 0) s[i] = -INFINITY;
  }
  if (st.m == -INFINITY) {
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) bm = fmaxf(bm, s[i] * sl2);
    st.m = fmaxf(bm, __shfl_xor(bm, 32));   // both lanes of a head
    st.seen = fmaxf(st.seen, st.m);
  }
  // The weights of the first K step of the value product (the lane's values i = 0..7) come
  // first; those of the second K step (i = 8..15), and the lane's logit maximum that a restart
  // needs, are computed between the first step's matrix instructions, and the overflow test
  // follows that step: a row that restarts discards its accumulators, so the first step's
  // products need not wait for the test.
  bf16x8 pb[2];
  float lsum = 0.f, smax = -INFINITY;
  const float nm = -st.m;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, nm));
    lsum += p;
    pb[0][i] = (__bf16)p;
  }
  // O^T[v, head] += V^T[v, keys] P^T[keys, head]. K step j covers keys 16j + 8h + 4g + jj
  // (h = 0, 1; jj = 0..3): the lane's P values i = 8j + 4h + jj. The V^T operand comes from two
  // transposing reads: lane (4jj + q) of each 16-lane group points at value dims
  // v0 = 32vt + 16*(group & 1) + 4q .. +3 of key 16j + 8h + 4g + jj.
  // chunk c = 4vt + 2grp + q/2: c/8 = vt/2, c%8 = 4(vt%2) + 2grp + q/2; key s = kbase + 16j + 8h
  // + 4g + jj: s/8 = kbase/8 + 2j + h, s%8 = 4g + jj, s%16 = 8h + 4g + jj. Slot (vt/2)*512 +
  // (s/8)*64 + (s%8)*8 + ((c%8) ^ kv_swz(s%16)), byte offset 8 * (q % 2) inside it.
  const int grp = (lane >> 4) & 1, li = lane & 15;
  const int jj = li >> 2, q4 = li & 3;
  const uint8_t* vb_lane = buf + ((kbase >> 3) * 64 + (4 * g + jj) * 8) * 16 + (q4 & 1) * 8;
  // 4 per-lane base addresses ([vt % 2][h]); every read is one of them plus an immediate offset
  const uint8_t* vb[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      vb[p][h] = vb_lane + h * 1024 + ((4 * p + 2 * grp + (q4 >> 1)) ^ kv_swz(8 * h + 4 * g + jj)) * 16;
  auto vop = [&](int step) -> bf16x8 {
    const int j = step / (MDV / 32), vt = step % (MDV / 32);
    const int off = (vt >> 1) * 8192 + j * 2048;
    const s16x4 lo = lds_read_tr16(vb[vt & 1][0] + off);
    const s16x4 hi = lds_read_tr16(vb[vt & 1][1] + off);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int NSTEP = 2 * (MDV / 32);
  bf16x8 va[VRING];
#pragma unroll
  for (int step = 0; step < VRING - 1; ++step) va[step] = vop(step);
#pragma unroll
  for (int step = 0; step < NSTEP; ++step) {
    if (step + VRING - 1 < NSTEP) va[(step + VRING - 1) % VRING] = vop(step + VRING - 1);
    const int j = step / (MDV / 32), vt = step % (MDV / 32);
    acc_o[vt] = mfma_bf16_32x32x16(va[step % VRING], pb[j], acc_o[vt]);
    if (step < 8) {   // second K step's weight i = 8 + step, running logit maximum
      const float p = __builtin_amdgcn_exp2f(fmaf(s[8 + step], sl2, nm));
      lsum += p;
      pb[1][step] = (__bf16)p;
      smax = fmaxf(smax, fmaxf(s[step], s[8 + step]));
    }
    if (step == MDV / 32 - 1) {
      const bool over = !(lsum <= 0x1p60f);
      if (__any(over)) {
        // the lane's maximum of sl2 * s (sl2 > 0: the product of the maximum, NaN ignored)
        const float lm = smax * sl2;
        const float hm = fmaxf(lm, __shfl_xor(lm, 32));
        st.seen = fmaxf(st.seen, hm);
        // with finite logits an overflowing lane always has a larger maximum to restart from,
        // and each restart raises some head's reference; NaN or infinite logits have none, and
        // their pass goes on (its output is then not finite) instead of restarting forever
        if (__any(over && hm > st.m)) return true;
      }
      st.l += lsum;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return false;
}

// One gathered block of 64 keys, processed as two halves. Returns true if the row must restart.
template <bool UT>
__device__ __forceinline__ bool attend_block(const uint8_t* buf, uint64_t vmask,
                                             const bf16x8 (&qreg)[MT], v16f (&acc_o)[MDV / 32],
                                             SoftmaxState& st, float sl2, int lane,
                                             uint8_t* gbuf, __amdgpu_buffer_rsrc_t seq, int ra, int rb,
                                             bool gon, int wave) {
  // the next block's gather goes out during this block's first computed half, one load every
  // other matrix instruction
  const __amdgpu_buffer_rsrc_t gseq = seq;
  uint8_t* const gdst = gbuf + (2 * wave) * 1024;
  const int gvoff0 = ra * (MDQK * 2) + ((lane & 7) ^ kv_swz(lane >> 3)) * 16;
  const int gvoff1 = rb * (MDQK * 2) + ((lane & 7) ^ kv_swz(8 | (lane >> 3))) * 16;
  bool pending = true;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    const uint32_t m32 = (uint32_t)(vmask >> (32 * h));
    if (m32) {
      const bool rs = attend_half<UT>(buf, 32 * h, m32, qreg, acc_o, st, sl2, lane, gseq,
                                  pending && gon ? gdst : nullptr, gvoff0, gvoff1);
      pending = false;
      if (rs) return true;
    }
  }
  if (pending && gon) gather_block<UT>(gbuf, seq, ra, rb, wave, lane);   // no half was computed
  return false;
}

// Stores a wave's output block, O^T in the accumulators (head c32 of the wave, values
// 32 vt + 8 i + 4 g + 0..3 in acc_o[vt][4 i .. 4 i + 3]), times inv, as bf16 rows dst + h * MDV
// (h = 0..31). The rows go through 32 KB of LDS (row h at h * 1024 bytes, its 16-byte chunk c at
// position c ^ (h % 16)), so that each global store writes one head's whole row (1 KB) instead
// of 16-byte pieces of 32 rows.
__device__ __forceinline__ void store_head_rows(uint16_t* dst, const v16f (&acc_o)[MDV / 32], float inv,
                                                uint8_t* stage, int lane) {
  const int g = lane >> 5, c32 = lane & 31;
  uint8_t* const mine = stage + c32 * (MDV * 2) + g * 8;
#pragma unroll
  for (int vt = 0; vt < MDV / 32; ++vt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 pk;
      pk.x = pack_bf16x2(acc_o[vt][4 * i4 + 0] * inv, acc_o[vt][4 * i4 + 1] * inv);
      pk.y = pack_bf16x2(acc_o[vt][4 * i4 + 2] * inv, acc_o[vt][4 * i4 + 3] * inv);
      *reinterpret_cast<uint2*>(mine + (((4 * vt + i4) ^ (c32 & 15)) * 16)) = pk;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // (one wave writes and reads its own rows: its LDS operations complete in order)
#pragma unroll 4
  for (int h = 0; h < 32; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(stage + h * (MDV * 2) + ((lane ^ (h & 15)) * 16));
    *reinterpret_cast<uint4*>(dst + (int64_t)h * MDV + 8 * lane) = v;
  }
}

// One workgroup per (query row, split of its index list): the row's entries are split into
// gridDim.y runs of whole blocks. A null idx stands for the list 0, 1, ..., pos, -1, ... (every
// causal candidate: the selection when a sequence has at most k keys). With one split the
// workgroup writes the normalised output and lse; with several it writes, per head, its
// normalised partial output and its partial log2-sum-exp to part_o [splits][T][H][d_v] (bf16)
// and part_lse [splits][T][H] (fp32), which attn_combine_kernel merges.
template <bool UT>
__global__ void __launch_bounds__(256, 1)
attn_bf16_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                 const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                 const int32_t* __restrict__ idx, int k, float scale, uint16_t* __restrict__ out,
                 float* __restrict__ lse, int T, uint16_t* __restrict__ part_o,
                 float* __restrict__ part_lse, int prefix_rows) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf0[MBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t buf1[MBUF];
  // restart requests: slot (step & 1) holds the id of the last step that asked for one
  __shared__ int s_flag[2];
  // rows from the last: in a causal batch the later rows of a sequence have more candidates, so
  // the heaviest start first and the short ones fill the tail
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 5, c32 = lane & 31;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int split = blockIdx.y, nsplit = gridDim.y;
  // Without an index list, entry e of a row is candidate e (e <= pos). With prefix_rows, a row
  // whose causal candidates all fit in k holds the list 0..pos, -1, ... (the selection of such a
  // row is every candidate, in ascending order) and is walked the same way. Such a row's blocks
  // end at its position; with an arbitrary list all k entries can be valid.
  const bool implicit = !idx || (prefix_rows && L.pos + 1 <= k);
  const int kr = implicit ? max(0, min(k, L.pos + 1)) : k;
  const int nblk_row = (kr + MBLK - 1) / MBLK;
  const int b0 = split * nblk_row / nsplit, b1 = (split + 1) * nblk_row / nsplit;
  // this split's entries
  const int32_t* ir = implicit ? nullptr : idx + (int64_t)r * k + b0 * MBLK;
  const int kk = min(kr - b0 * MBLK, (b1 - b0) * MBLK);
  const int nblk = b1 - b0;

  // lane l's key of block blk is entry blk*64 + l of the index row
  auto load_idx = [&](int blk) -> int {
    const int j = blk * MBLK + lane;
    if (blk >= nblk || j >= kk) return -1;
    if (ir) return ir[j];
    const int e = b0 * MBLK + j;
    return e <= L.pos ? e : -1;
  };
  // the first block's entries are requested before the query block, so that the first gather
  // waits for them only (a decode workgroup has few blocks to hide this start-up behind)
  const int idx_first = load_idx(0);

  // query block of this wave as B operand: head 32w + c32, dims 16t + 8g .. +8
  bf16x8 qreg[MT];
  {
    const uint16_t* qh = q + ((int64_t)r * MH + 32 * wave + c32) * MDQK + 8 * g;
#pragma unroll
    for (int t = 0; t < MT; ++t) qreg[t] = *reinterpret_cast<const bf16x8*>(qh + 16 * t);
  }
  v16f acc_o[MDV / 32];
  SoftmaxState st{-INFINITY, -INFINITY, 0.f};
  const float sl2 = scale * 1.4426950408889634f;
  if (threadIdx.x == 0) s_flag[0] = s_flag[1] = -1;
  // the sequence's latent rows as a buffer (byte offsets fit 32 bits: n * 1152 < 2^31 is checked
  // on the host); out-of-range offsets would read as zero
  const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kv + (int64_t)L.kofs * (MDQK * 2)), 0, L.n * (MDQK * 2), 0x00020000);
  // sequence-local rows of keys 16w + l/8 and 16w + 8 + l/8 (see gather_block) and the block's
  // valid mask
  auto prep = [&](int sidx, int& ra, int& rb, uint64_t& vm) {
    const bool valid = sidx >= 0 && sidx < L.n;
    vm = __ballot(valid);
    const int row = valid ? sidx : 0;
    ra = __shfl(row, 16 * wave + (lane >> 3));
    rb = __shfl(row, 16 * wave + 8 + (lane >> 3));
  };

  // Pipeline: wait for the block in flight, barrier (its LDS data is complete and every wave
  // has finished with the other buffer), start gathering the next block into the other buffer,
  // then compute on the current one while that gather is in flight.
  // A wave that needs a restart records it in s_flag[step & 1] = step (before the next barrier);
  // every wave reads the previous step's slot right after that barrier, so all waves agree.
  int step = 0;
  int ra, rb;
  uint64_t vm_cur, vm_next;
  prep(idx_first, ra, rb, vm_cur);
  if (vm_cur) gather_block<UT>(buf0, seq, ra, rb, wave, lane);
  for (;;) {
#pragma unroll
    for (int vt = 0; vt < MDV / 32; ++vt) acc_o[vt] = (v16f){};
    st.m = st.seen;  // -inf on the first pass, the largest recorded half maximum on a restart
    st.l = 0.f;
    int idx_next = load_idx(1);
    bool restart = false;
    for (int blk = 0; blk < nblk; blk += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (blk > 0 && s_flag[(step - 1) & 1] == step - 1) { restart = true; break; }
      prep(idx_next, ra, rb, vm_next);
      const bool gon1 = blk + 1 < nblk && vm_next;
      idx_next = load_idx(blk + 2);
      // (a block without a valid key skips both halves but still issues the second loads)
      if (attend_block<UT>(buf0, vm_cur, qreg, acc_o, st, sl2, lane, buf1, seq, ra, rb, gon1, wave)) s_flag[step & 1] = step;
      ++step;
      vm_cur = vm_next;
      if (blk + 1 >= nblk) break;

      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (s_flag[(step - 1) & 1] == step - 1) { restart = true; break; }
      prep(idx_next, ra, rb, vm_next);
      const bool gon0 = blk + 2 < nblk && vm_next;
      idx_next = load_idx(blk + 3);
      // (a block without a valid key skips both halves but still issues the second loads)
      if (attend_block<UT>(buf1, vm_cur, qreg, acc_o, st, sl2, lane, buf0, seq, ra, rb, gon0, wave)) s_flag[step & 1] = step;
      ++step;
      vm_cur = vm_next;
    }
    // a request made during the last step is visible after one more barrier (a split without a
    // block, step 0, has made none: the flags' initial -1 must not read as step -1's request)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!restart && step > 0 && s_flag[(step - 1) & 1] == step - 1) restart = true;
    if (!restart) break;
    // restart: gather the first block again
    prep(load_idx(0), ra, rb, vm_cur);
    if (vm_cur) gather_block<UT>(buf0, seq, ra, rb, wave, lane);
  }

  // finish: combine the two lane halves' sums (same head), normalise, store (the block buffers
  // are free after the last barrier: each wave stages its 32 heads' rows in 32 KB of them)
  const float ltot = st.l + __shfl_xor(st.l, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const int head = 32 * wave + c32;
  uint8_t* const stage = (wave < 2 ? buf0 : buf1) + (wave & 1) * (32 * MDV * 2);
  const int64_t rh = ((int64_t)(nsplit > 1 ? split * T : 0) + r) * MH + head;
  store_head_rows((nsplit > 1 ? part_o : out) + (rh - c32) * MDV, acc_o, inv, stage, lane);
  if (g == 0) {
    // log2-sum-exp (-inf for no valid entry, NaN after non-finite logits)
    const float l2 = ltot == 0.f ? -INFINITY : st.m + __log2f(ltot);
    if (nsplit > 1) part_lse[rh] = l2;
    else if (lse) lse[rh] = l2 * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------------------- alignment target
// Indexer-alignment target (page "DeepSeek-V3.2: Pushing the Frontier of Open Large Language
// Models" (paper digest), sections "Key claims" (paper section 2.1.1, Eq. 3-4) and "Method": the
// indexer learns, through a KL loss, the main attention's distribution aggregated over the
// heads, over all preceding keys or the selected ones). For query row r and its index list
// (entries outside 0..pos skipped, repeats counted as listed):
//   p[e]  = (1/H) sum_h exp(z_{h,e} - lse_h),   z_{h,e} = scale * q[r,h] . kv[row s_e]
//   KL[r] = sum_e p[e] * (ln p[e] - ln softmax_e(I[r, s_e]))
// with lse the attention's log-sum-exp over the same entries. One workgroup per row, two per
// compute unit: the indexer normaliser first (two block reductions over the listed scores), then
// the latent rows stream through one LDS block buffer laid out as the attention's; per half
// block each wave computes
// the logits of its 32 heads on the matrix core (as the attention does), turns them into
// probabilities against the given lse, and sums them over its heads with a reduce-scatter across
// lanes; the four waves' sums meet in LDS, where the first wave forms p and the KL terms.

__device__ __forceinline__ float block_reduce_256(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float t = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, t) : v + t;
  }
  __syncthreads();   // red is free (earlier readers are done)
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

// Logits of one half block for the wave's heads (same operand layout as attend_half); with gdst
// set, the next block's gather goes out one load every other matrix instruction (as there).
__device__ __forceinline__ v16f half_logits(const uint8_t* buf, int kbase, const bf16x8 (&qreg)[MT],
                                            int lane, __amdgpu_buffer_rsrc_t gseq, uint8_t* gdst,
                                            int gvoff0, int gvoff1) {
  const int g = lane >> 5, c32 = lane & 31;
  const uint8_t* kb_lane = buf + (((kbase + c32) >> 3) * 64 + (c32 & 7) * 8) * 16;
  const int ksw = kv_swz(c32 & 15);
  const uint8_t* kb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) kb[q] = kb_lane + ((2 * q + g) ^ ksw) * 16;
  auto kop = [&](int t) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(kb[t & 3] + (t >> 2) * 8192);
  };
  v16f s = {};
  bf16x8 ka[KRING];
#pragma unroll
  for (int t = 0; t < KRING - 1; ++t) ka[t] = kop(t);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t + KRING - 1 < MT) ka[(t + KRING - 1) % KRING] = kop(t + KRING - 1);
    s = mfma_bf16_32x32x16(ka[t % KRING], qreg[t], s);
    if ((t & 1) == 0 && gdst)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          gseq, (__attribute__((address_space(3))) void*)(gdst + ((t / 2) / 9) * 1024 + ((t / 2) % 9) * 8192),
          16, (t / 2) / 9 ? gvoff1 : gvoff0, ((t / 2) % 9) * 128, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

__global__ void __launch_bounds__(256, 2)
align_bf16_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                  const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                  const int32_t* __restrict__ idx, int k, float scale, const float* __restrict__ lse,
                  const float* __restrict__ scores, int64_t ld, float* __restrict__ target,
                  float* __restrict__ kl) {
  // one block buffer (72 KB), so that two rows share a compute unit: one row's gather overlaps
  // the other's matrix work
  __shared__ __attribute__((aligned(1024))) uint8_t buf[MBUF];
  __shared__ float psum[2][4][MBLK];   // per block parity and wave: head sums of the block's keys
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int32_t* ir = idx + (int64_t)r * k;
  const float* srow = scores + (int64_t)r * ld;
  float* trow = target ? target + (int64_t)r * k : nullptr;
  auto valid_entry = [&](int s) { return s >= 0 && s <= L.pos; };

  // 1. ln of the indexer softmax normaliser over the valid entries
  float mx = -INFINITY;
  for (int e = tid; e < k; e += 256) {
    const int s = ir[e];
    if (valid_entry(s)) mx = fmaxf(mx, srow[s]);
  }
  mx = block_reduce_256(mx, red, true);
  if (mx == -INFINITY) {   // uniform: no valid entry
    if (trow)
      for (int e = tid; e < k; e += 256) trow[e] = 0.f;
    if (tid == 0) kl[r] = 0.f;
    return;
  }
  float se = 0.f;
  for (int e = tid; e < k; e += 256) {
    const int s = ir[e];
    if (valid_entry(s)) se += __expf(srow[s] - mx);
  }
  se = block_reduce_256(se, red, false);
  const float lnz = mx + __logf(se);

  // 2. query block of this wave (head 32w + c32) and the head's lse (log2 domain)
  bf16x8 qreg[MT];
  {
    const uint16_t* qh = q + ((int64_t)r * MH + 32 * wave + c32) * MDQK + 8 * g;
#pragma unroll
    for (int t = 0; t < MT; ++t) qreg[t] = *reinterpret_cast<const bf16x8*>(qh + 16 * t);
  }
  const float sl2 = scale * 1.4426950408889634f;
  const float nl2 = -lse[(int64_t)r * MH + 32 * wave + c32] * 1.4426950408889634f;
  const int nblk = (k + MBLK - 1) / MBLK;
  const __amdgpu_buffer_rsrc_t seq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(kv + (int64_t)L.kofs * (MDQK * 2)), 0, L.n * (MDQK * 2), 0x00020000);
  auto load_idx = [&](int blk) -> int {
    const int j = blk * MBLK + lane;
    return (blk < nblk && j < k) ? ir[j] : -1;
  };
  auto prep = [&](int sidx, int& ra, int& rb, uint64_t& vm) {
    const bool v = valid_entry(sidx);
    vm = __ballot(v);
    const int row = v ? sidx : 0;
    ra = __shfl(row, 16 * wave + (lane >> 3));
    rb = __shfl(row, 16 * wave + 8 + (lane >> 3));
  };
  int ra, rb;
  uint64_t vm_cur, vm_next;
  int sidx_cur = load_idx(0);
  prep(sidx_cur, ra, rb, vm_cur);
  if (vm_cur) gather_block<false>(buf, seq, ra, rb, wave, lane);
  int sidx_next = load_idx(1);
  float klacc = 0.f;   // first wave: this lane's KL terms
  // the first wave forms p and the KL terms of a block after the next barrier (the waves' head
  // sums of block b sit in psum[b & 1]); its entry's index and validity are kept until then
  int sidx_prev = -1;
  bool ok_prev = false, have_prev = false;
  auto finish_prev = [&](int pblk) {
    if (wave == 0 && have_prev) {
      const int e = pblk * MBLK + lane;
      const float p = ok_prev ? (psum[pblk & 1][0][lane] + psum[pblk & 1][1][lane] + psum[pblk & 1][2][lane] +
                                 psum[pblk & 1][3][lane]) * (1.f / MH)
                              : 0.f;
      if (trow && e < k) trow[e] = p;
      if (p > 0.f) klacc += p * (__logf(p) - (srow[sidx_prev] - lnz));
    }
  };

  for (int blk = 0; blk < nblk; ++blk) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // the block is in LDS; the previous block's head sums are complete
    finish_prev(blk - 1);
    prep(sidx_next, ra, rb, vm_next);
    const bool gon = blk + 1 < nblk && vm_next;
    const int sidx_after = load_idx(blk + 2);
    if (vm_cur) {   // uniform
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        const uint32_t m32 = (uint32_t)(vm_cur >> (32 * h));
        if (!m32) continue;   // uniform; its keys are skipped when the block is finished
        const v16f sv = half_logits(buf, 32 * h, qreg, lane, seq, nullptr, 0, 0);
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int b = 8 * (i >> 2) + (i & 3);
          const uint64_t lanes = (((m32 >> b) & 1u) ? 0x00000000FFFFFFFFull : 0ull) |
                                 (((m32 >> (b + 4)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
          v[i] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, nl2)) : 0.f;
        }
        // sum over the 32 heads of the wave (lanes of equal g): reduce-scatter; lane bits
        // (16, 8, 4, 2) pick value index 8*b16 + 4*b8 + 2*b4 + b2, the last step adds lane pairs.
        // Partner values by lane-xor: swizzles (xor 16, 4) and row-local moves (xor 8, 2, 1).
        auto xor16 = [](float x) { return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1F)); };
        auto xor4 = [](float x) { return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F)); };
        auto xor8 = [](float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)); };
        auto xor2 = [](float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)); };
        auto xor1 = [](float x) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)); };
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool hi = (lane & 16) != 0;
          const float keep = hi ? v[j + 8] : v[j], give = hi ? v[j] : v[j + 8];
          v[j] = keep + xor16(give);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool hi = (lane & 8) != 0;
          const float keep = hi ? v[j + 4] : v[j], give = hi ? v[j] : v[j + 4];
          v[j] = keep + xor8(give);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bool hi = (lane & 4) != 0;
          const float keep = hi ? v[j + 2] : v[j], give = hi ? v[j] : v[j + 2];
          v[j] = keep + xor4(give);
        }
        {
          const bool hi = (lane & 2) != 0;
          const float keep = hi ? v[1] : v[0], give = hi ? v[0] : v[1];
          v[0] = keep + xor2(give);
        }
        v[0] += xor1(v[0]);
        if ((lane & 1) == 0) {
          const int i = 8 * ((lane >> 4) & 1) + 4 * ((lane >> 3) & 1) + 2 * ((lane >> 2) & 1) + ((lane >> 1) & 1);
          psum[blk & 1][wave][32 * h + 8 * (i >> 2) + 4 * g + (i & 3)] = v[0];
        }
      }
    }
    __syncthreads();   // every wave is done with the buffer
    if (gon) gather_block<false>(buf, seq, ra, rb, wave, lane);
    have_prev = true;
    ok_prev = (vm_cur >> lane) & 1ull;
    sidx_prev = sidx_cur;
    vm_cur = vm_next;
    sidx_cur = sidx_next;
    sidx_next = sidx_after;
  }
  __syncthreads();   // the last block's head sums
  finish_prev(nblk - 1);
  if (wave == 0) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) klacc += __shfl_xor(klacc, o);
    if (lane == 0) kl[r] = klacc;
  }
}

hipError_t launch_align_bf16(const SeqInfo& s, const uint16_t* q, const uint16_t* kv,
                             const int32_t* idx, int k, float scale, const float* lse,
                             const float* scores, int64_t ld, float* target, float* kl,
                             hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  hipLaunchKernelGGL(align_bf16_kernel, dim3(s.T), dim3(256), 0, st, s.B, s.cu_q, s.cu_k, q,
                     reinterpret_cast<const uint8_t*>(kv), idx, k, scale, lse, scores, ld, target, kl);
  return hipGetLastError();
}

// Merges the splits of one (row, head) per wave: with M the largest partial log2-sum-exp, split
// s weighs 2^(lse_s - M); out = sum of weighted partial outputs / sum of weights, lse = M +
// log2(sum of weights) (natural log on output). Splits without a valid entry have weight 0; a
// row without any gives out = 0, lse = -inf.
__global__ void __launch_bounds__(256)
attn_combine_kernel(int T, int nsplit, const uint16_t* __restrict__ part_o,
                    const float* __restrict__ part_lse, uint16_t* __restrict__ out,
                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // row * H + head
  if (rh >= (int64_t)T * MH) return;
  const int64_t stride = (int64_t)T * MH;
  // the first four splits' partial rows are requested together with the log2-sum-exps, before
  // the weights are known: one memory round trip for up to four splits (every split writes its
  // rows, an empty one zeros; steps past the last split re-read split 0 with weight 0)
  auto load4 = [&](int sp, uint4 (&pk)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s2 = sp + i < nsplit ? sp + i : 0;
      pk[i] = *reinterpret_cast<const uint4*>(part_o + (s2 * stride + rh) * MDV + 8 * lane);
    }
  };
  uint4 pk0[4];
  load4(0, pk0);
  // lane s < nsplit holds split s's log2-sum-exp (nsplit <= 32)
  const float my_ls = lane < nsplit ? part_lse[lane * stride + rh] : -INFINITY;
  float M = my_ls;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const bool nan_part = __any(my_ls != my_ls);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    // four splits per step (an empty split weighs 2^-inf = 0)
    for (int sp = 0; sp < nsplit; sp += 4) {
      uint4 pk[4];
      float w[4];
      if (sp == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pk0[i];
      } else {
        load4(sp, pk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = sp + i < nsplit ? __builtin_amdgcn_exp2f(__shfl(my_ls, sp + i) - M) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wsum += w[i];
        const uint32_t wd[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += w[i] * __uint_as_float(wd[j] << 16);
          acc[2 * j + 1] += w[i] * __uint_as_float(wd[j] & 0xFFFF0000u);
        }
      }
    }
  }
  // a NaN partial (non-finite logits in that split) makes the head's output and lse NaN
  const float inv = nan_part ? __builtin_nanf("") : wsum > 0.f ? 1.f / wsum : 0.f;
  uint4 pk;
  pk.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  pk.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  pk.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(out + rh * MDV + 8 * lane) = pk;
  if (lse && lane == 0)
    lse[rh] = nan_part ? __builtin_nanf("") : wsum > 0.f ? (M + __log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

// Splits of each row's index list: batches with fewer rows than compute units (decode) split
// every row into up to 32 runs of whole blocks so that each compute unit gets a workgroup.
// A function of the arguments only (the workspace size depends on it).
int attn_splits(const SeqInfo& s, int k) {
  const int nblk = (k + MBLK - 1) / MBLK;
  if (s.T <= 0 || s.T >= kTargetCUs) return 1;
  return max(1, min(min(nblk, 32), kTargetCUs / s.T));
}

size_t attn_workspace_bytes(const SeqInfo& s, int, int, int, int k, bool bf16) {
  if (!bf16) return 0;
  const int ns = attn_splits(s, k);
  return ns > 1 ? (size_t)ns * s.T * MH * (MDV * sizeof(uint16_t) + sizeof(float)) : 0;
}

hipError_t launch_attn_bf16(const SeqInfo& s, const uint16_t* q, const uint16_t* kv,
                            const int32_t* idx, int k, float scale, uint16_t* out, float* lse,
                            void* ws, size_t, bool prefix_rows, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int ns = attn_splits(s, k);
  uint16_t* part_o = ns > 1 ? static_cast<uint16_t*>(ws) : nullptr;
  float* part_lse = ns > 1 ? reinterpret_cast<float*>(part_o + (size_t)ns * s.T * MH * MDV) : nullptr;
  if (ns > 1)
    hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3(s.T, ns), dim3(256), 0, st, s.B, s.cu_q, s.cu_k, q,
                       reinterpret_cast<const uint8_t*>(kv), idx, k, scale, out, lse, s.T, part_o,
                       part_lse, prefix_rows ? 1 : 0);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3(s.T, ns), dim3(256), 0, st, s.B, s.cu_q, s.cu_k, q,
                       reinterpret_cast<const uint8_t*>(kv), idx, k, scale, out, lse, s.T, part_o,
                       part_lse, prefix_rows ? 1 : 0);
  if (ns > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3((s.T * MH + 3) / 4), dim3(256), 0, st, s.T, ns,
                       part_o, part_lse, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
