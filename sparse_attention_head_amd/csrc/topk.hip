// Causal per-row top-k selection on gfx950.
//
// For each query row: the min(k, pos+1) positions s <= pos with the largest index scores
// (36kr article, section "02. Built on the final version of DeepSeek-V3.1": retrieve only the
// entries with the top-k index scores; paper digest, "Key claims", paper section 2.1, Eq. 2).
// Ties prefer the lower position, +0 equals -0, output ascending and padded with -1.
//
// Method (exact, deterministic): scores map to order-preserving 32-bit keys. A radix select over
// the key digits (11, 11 and 10 bits, most significant first) finds the k-th largest key T and the
// number `need` of keys equal to T that belong to the selection. An ordered compaction pass then
// keeps, in position order, every key > T and the first `need` keys == T; its output is ascending
// by construction. Per tile of the row, the prefix counts come from wavefront ballots
// (mbcnt-style popcounts) plus one small exchange across waves.
#include "dsa_internal.h"
#include "device_common.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

__global__ void __launch_bounds__(TK_THREADS)
topk_row_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t xch[2][TK_WAVES][2];
  __shared__ uint32_t s_digit, s_above;

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int n = L.pos + 1;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;

  if (n <= k) {  // every candidate is selected
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }

  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)k;  // how many of the keys matching `prefix` still go in
  const int n4 = n & ~3;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = tid * 4; i < n4; i += TK_THREADS * 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + i);
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = float_to_ordered(e[j]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
      }
    }
    for (int i = n4 + tid; i < n; i += TK_THREADS) {
      const uint32_t u = float_to_ordered(row[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // suffix sums over the bins (from the largest digit down) to find the bin of the
      // need-th largest key among those matching the prefix
      const int per = nb / 64;
      uint32_t sum = 0;
      for (int j = 0; j < per; ++j) sum += hist[lane * per + j];
      uint32_t suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_down(suf, off);
        if (lane + off < 64) suf += t;
      }
      const uint32_t above_lane = suf - sum;  // keys in bins of higher lanes
      if (suf >= need && above_lane < need) {
        uint32_t above = above_lane;
        for (int j = per - 1; j >= 0; --j) {
          const uint32_t h = hist[lane * per + j];
          if (above + h >= need) {
            s_digit = (uint32_t)(lane * per + j);
            s_above = above;
            break;
          }
          above += h;
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    need -= s_above;
  }
  const uint32_t T = prefix;  // the k-th largest key; `need` >= 1 keys equal to T are taken

  // ordered compaction: selected before i = (# keys > T before i) + min(# keys == T before i, need)
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0, it = 0; base < n; base += TK_THREADS, ++it) {
    const int i = base + tid;
    const uint32_t u = i < n ? float_to_ordered(row[i]) : 0u;
    const bool gt = i < n && u > T;
    const bool eq = i < n && u == T;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    const int par = it & 1;
    if (lane == 0) {
      xch[par][wave][0] = (uint32_t)__popcll(bgt);
      xch[par][wave][1] = (uint32_t)__popcll(beq);
    }
    __syncthreads();
    uint32_t gt_before = run_gt + lanes_below(bgt), eq_before = run_eq + lanes_below(beq);
    uint32_t tot_gt = 0, tot_eq = 0;
    for (int v = 0; v < TK_WAVES; ++v) {
      const uint32_t a = xch[par][v][0], b2 = xch[par][v][1];
      if (v < wave) { gt_before += a; eq_before += b2; }
      tot_gt += a;
      tot_eq += b2;
    }
    const uint32_t at = gt_before + min(eq_before, need);
    if ((gt || (eq && eq_before < need)) && at < (uint32_t)k) out[at] = i;
    run_gt += tot_gt;
    run_eq += tot_eq;
    if (run_gt + min(run_eq, need) >= (uint32_t)k) break;  // uniform: all k written
  }
}

size_t topk_workspace_bytes(const SeqInfo&, int) { return 0; }

hipError_t launch_topk(const SeqInfo& s, const float* scores, int64_t ld, int k, int32_t* idx,
                       void*, size_t, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_row_kernel, dim3(s.T), dim3(TK_THREADS), 0, st, s.B, s.cu_q, s.cu_k,
                     scores, ld, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
