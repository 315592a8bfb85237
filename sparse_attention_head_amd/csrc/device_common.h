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

// Largest b with cu[b] <= r (cu is non-decreasing, cu[0] = 0 <= r < cu[B]).
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (__ldg(cu + mid) <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

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
