// Device-side helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Where a query row sits: sequence b, its causal position pos = n_b - m_b + i, the first key
// row of the sequence and the sequence's key count.
struct RowLoc {
  int b;
  int pos;
  int kofs;
  int n;
};

// Largest b with cu[b] <= r (cu is non-decreasing, cu[0] = 0 <= r < cu[B]; r wave-uniform). All
// 64 lanes of the wave take part: each round tests 64 evenly spaced candidates at once (the true
// ones are a prefix of the lanes), so a batch of up to 64 sequences costs one round of loads where
// a binary search would chain log2(B) dependent loads.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int B, int r) {
  const int lane = (int)__lane_id();
  int lo = 0, hi = B - 1;   // invariant: cu[lo] <= r < cu[hi + 1]
  while (lo < hi) {
    const int step = (hi - lo + 63) >> 6;   // >= 1
    const int p = lo + (lane + 1) * step;   // candidates lo + step .. lo + 64 step
    const bool t = p <= hi && __ldg(cu + p) <= r;
    lo += __popcll(__ballot(t)) * step;     // the largest true candidate (or lo)
    hi = min(hi, lo + step - 1);            // the next candidate is false or beyond hi
  }
  return lo;
}

// (every lane of the wave calls it: see find_seq)
__device__ __forceinline__ RowLoc locate_row(const int32_t* __restrict__ cu_q,
                                             const int32_t* __restrict__ cu_k, int B, int r) {
  RowLoc L;
  // skip empty sequences: the last b with cu_q[b] <= r has cu_q[b+1] > r
  L.b = find_seq(cu_q, B, r);
  int q0 = __ldg(cu_q + L.b), q1 = __ldg(cu_q + L.b + 1);
  int k0 = __ldg(cu_k + L.b), k1 = __ldg(cu_k + L.b + 1);
  L.kofs = k0;
  L.n = k1 - k0;
  L.pos = L.n - (q1 - q0) + (r - q0);
  return L;
}

// Order-preserving map of a float to uint32 (larger float -> larger key), with -0 folded onto +0
// so that the two zeros tie.
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------- wave / block primitives

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

__device__ __forceinline__ uint32_t lanes_below_count(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave: four shifts within each row of 16 lanes,
// then each row's total broadcast into the rows above it (GCN data-parallel primitives).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Finds the bin holding the need-th largest key among the counted ones (nb bins, a power of two
// <= 2048; suffix sums from the top bin down). Called by all threads; wave 0 does the work: lane l
// sums bins l*per .. l*per + per - 1 (read in a lane-rotated order, which spreads the lanes over
// the banks), suffix sums across lanes (total minus a prefix scan) find the lane whose run holds
// the need-th largest key, and a second scan over that run's bins (one bin per lane) finds the
// bin.
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nb, uint32_t need,
                                           uint32_t* s_digit, uint32_t* s_above) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int per = nb >= 64 ? nb >> 6 : 1;
    uint32_t sum = 0;
    if (lane * per < nb)
      for (int j = 0; j < per; ++j) sum += hist[lane * per + ((j + lane) & (per - 1))];
    const uint32_t pre = wave_incl_scan(sum);
    const uint32_t total = __builtin_amdgcn_readlane(pre, 63);
    const uint32_t suf = total - pre + sum;   // bins of this lane and above
    const uint32_t above_lane = suf - sum;
    // the crossing lane: its run holds the need-th largest key
    const uint64_t hit = __ballot(suf >= need && above_lane < need);
    const int cl = __builtin_amdgcn_readfirstlane(hit ? (int)(__ffsll((unsigned long long)hit) - 1) : 0);
    const uint32_t above = __builtin_amdgcn_readlane(above_lane, cl);
    // bins of that run, one per lane (lane j: bin cl*per + j), suffix sums within the run
    const int bin = cl * per + lane;
    const uint32_t h = (lane < per && bin < nb) ? hist[bin] : 0u;
    const uint32_t pre2 = wave_incl_scan(h);
    const uint32_t rs = __builtin_amdgcn_readlane(pre2, 63) - pre2 + h;
    // the bin: above + (bins of the run above it) < need <= above + rs
    const uint64_t hb = __ballot(lane < per && above + rs >= need && above + rs - h < need);
    if (hb && lane == (int)(__ffsll((unsigned long long)hb) - 1)) {
      *s_digit = (uint32_t)bin;
      *s_above = above + rs - h;
    }
  }
  __syncthreads();
}


// ---------------------------------------------------------------------------- LDS DMA

// One 16-byte-per-lane LDS DMA (buffer_load_dwordx4 ... lds): lane i's 16 bytes at voffset +
// soff of the resource land at LDS byte address lds_base + lds_off + 16 i (lds_base, lds_off and
// soff wave-uniform). Written as inline assembly so that the compiler does not track it: its
// waits for LDS DMA are per LDS variable, so a read of one buffer would wait for DMAs still in
// flight into another (in the attention, the value product of the current block would wait for
// the next block's gather, an HBM round trip in decode). The callers wait for the DMA themselves
// (s_waitcnt vmcnt, counting the vector memory operations issued after it, which complete in
// order) and, when other waves read the data, synchronise. M0 is saved and restored around it,
// one wait state after its write (the hazard the compiler observes for its own LDS DMA) and one
// before its restore.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, int lds_off,
                                          int voff, int soff) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %4, %5 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "scc");
}

// LDS byte address of a shared-memory pointer, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

}  // namespace dsa
