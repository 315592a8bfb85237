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

// Maps a block index so that consecutive logical tiles land on the same XCD: the hardware
// dispatches workgroup i to XCD i % 8, so logical tile = xcd * per_xcd + slot.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  int per = nblocks / NX, rem = nblocks % NX;
  int xcd = bid % NX, slot = bid / NX;
  // the first `rem` XCDs get one extra tile
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

}  // namespace dsa
