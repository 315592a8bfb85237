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

// ------------------------------------------------------------------------------------------
// Register-resident variant for rows of up to 4096 * NT candidates. The row is read once, as
// float4: in tile j (positions 4096j .. 4096j + 4095) thread t holds positions 4096j + 4t + c,
// c = 0..3, and keeps only the upper 16 bits of their keys, two per register. Digits 1 and 2 of
// the threshold (key bits 31..21 and 20..16) come from registers; digits 3 and 4 (bits 15..8 and
// 7..0) only concern keys whose upper half equals the threshold's, and those few are re-read from
// memory. The ordered compaction counts, per lane, the keys above / equal to the threshold, scans
// the counts across the wave, stores one total per (tile, wave), turns those totals into offsets
// with one block-wide exclusive scan in (tile, wave) order -- which is position order -- and
// writes every selected position at its offset.

__device__ __forceinline__ uint32_t block_excl_scan2(uint32_t a, uint32_t b, uint32_t* sw,
                                                     uint32_t& excl_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t xa = a, xb = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t ta = __shfl_up(xa, off), tb = __shfl_up(xb, off);
    if (lane >= off) { xa += ta; xb += tb; }
  }
  if (lane == 63) { sw[2 * wave] = xa; sw[2 * wave + 1] = xb; }
  __syncthreads();
  uint32_t ba = 0, bb = 0;
  for (int w = 0; w < wave; ++w) { ba += sw[2 * w]; bb += sw[2 * w + 1]; }
  excl_b = bb + xb - b;
  return ba + xa - a;
}

// Inclusive scan of two small counts across the wave (packed in one 32-bit value).
__device__ __forceinline__ uint32_t wave_incl_scan_packed(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(x, off);
    if (lane >= off) x += t;
  }
  return x;
}

// Finds the bin holding the need-th largest key among the counted ones (suffix sums from the
// top bin down). Called by all threads; wave 0 does the work.
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nb, uint32_t need,
                                           uint32_t* s_digit, uint32_t* s_above) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int per = (nb + 63) / 64;
    uint32_t sum = 0;
    for (int j = 0; j < per; ++j) {
      const int bin = lane * per + j;
      sum += bin < nb ? hist[bin] : 0u;
    }
    uint32_t suf = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_down(suf, off);
      if (lane + off < 64) suf += t;
    }
    const uint32_t above_lane = suf - sum;
    if (suf >= need && above_lane < need) {
      uint32_t above = above_lane;
      for (int j = per - 1; j >= 0; --j) {
        const int bin = lane * per + j;
        const uint32_t h = bin < nb ? hist[bin] : 0u;
        if (above + h >= need) {
          *s_digit = (uint32_t)bin;
          *s_above = above;
          break;
        }
        above += h;
      }
    }
  }
  __syncthreads();
}

constexpr int TK_TILE = 4 * TK_THREADS;  // positions per tile

template <int NT>
__global__ void __launch_bounds__(TK_THREADS)
topk_reg_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx) {
  constexpr int NM = (4 * NT + 31) / 32;     // 32-bit words of per-thread position masks
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cnt[NT * TK_WAVES][2];  // per (tile, wave): keys > T, keys == T
  __shared__ uint32_t sw[2 * TK_WAVES];
  __shared__ uint32_t s_digit, s_above;

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int n = L.pos + 1;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;

  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const int tiles = (n + TK_TILE - 1) / TK_TILE;  // <= NT

  // Upper key halves: hk[2j] holds positions c = 0, 1 of tile j, hk[2j+1] c = 2, 3. Positions
  // past the end of the row get key 0, below the key of every finite float (whose top 11 bits
  // are >= 4), so they never reach the selection and need no bound checks later.
  uint32_t hk[2 * NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int e = j * TK_TILE + 4 * tid;
    uint32_t k4[4] = {0u, 0u, 0u, 0u};
    if (j < tiles) {
      if (e + 3 < n) {
        const float4 v = *reinterpret_cast<const float4*>(row + e);
        k4[0] = float_to_ordered(v.x);
        k4[1] = float_to_ordered(v.y);
        k4[2] = float_to_ordered(v.z);
        k4[3] = float_to_ordered(v.w);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < n) k4[c] = float_to_ordered(row[e + c]);
      }
    }
    hk[2 * j] = (k4[0] >> 16) | (k4[1] & 0xFFFF0000u);
    hk[2 * j + 1] = (k4[2] >> 16) | (k4[3] & 0xFFFF0000u);
    // opaque from here on: later digit extractions must use the packed halves, not the full
    // keys (which the compiler would otherwise keep alive)
    asm volatile("" : "+v"(hk[2 * j]), "+v"(hk[2 * j + 1]));
    if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the loads in flight
  }
#define HI(j, c) ((hk[2 * (j) + ((c) >> 1)] >> (16 * ((c) & 1))) & 0xFFFFu)

  uint32_t need = (uint32_t)k;
  // digit 1: key bits 31..21 = upper-half bits 15..5
  for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NT; ++j)
    if (j < tiles)
#pragma unroll
      for (int c = 0; c < 4; ++c) atomicAdd(&hist[HI(j, c) >> 5], 1u);
  __syncthreads();
  select_bin(hist, 2048, need, &s_digit, &s_above);
  const uint32_t d1 = s_digit;
  need -= s_above;
  __syncthreads();
  // digit 2: key bits 20..16 among upper halves whose digit 1 is d1
  if (tid < 32) hist[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NT; ++j)
    if (j < tiles)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((HI(j, c) >> 5) == d1) atomicAdd(&hist[HI(j, c) & 31u], 1u);
  __syncthreads();
  select_bin(hist, 32, need, &s_digit, &s_above);
  const uint32_t P16 = (d1 << 5) | s_digit;
  need -= s_above;
  __syncthreads();

  // positions whose upper half equals P16 (bit 4j + c): only these need their low halves
  uint32_t tie[NM];
#pragma unroll
  for (int w = 0; w < NM; ++w) tie[w] = 0u;
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (HI(j, c) == P16) tie[(4 * j + c) >> 5] |= 1u << ((4 * j + c) & 31);
  const float* mine = row + 4 * tid;  // position of bit b: (b / 4) * TK_TILE + 4 * tid + b % 4
  // digits 3 and 4: bits 15..8 and 7..0 of those keys, re-read from memory (few of them)
  uint32_t lo_prefix = 0, lo_mask = 0;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 8 : 0;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < NM; ++w) {
      uint32_t m = tie[w];
      while (m) {
        const int bit = 32 * w + __ffs(m) - 1;
        m &= m - 1;
        const uint32_t lo = float_to_ordered(mine[(bit >> 2) * TK_TILE + (bit & 3)]) & 0xFFFFu;
        if ((lo & lo_mask) == lo_prefix) atomicAdd(&hist[(lo >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    select_bin(hist, 256, need, &s_digit, &s_above);
    lo_prefix |= s_digit << shift;
    lo_mask |= 255u << shift;
    need -= s_above;
    __syncthreads();
  }
  const uint32_t T = (P16 << 16) | lo_prefix;  // the k-th largest key; `need` keys == T go in

  // classes of the tied positions: above T / equal to T
  uint32_t tgt[NM], teq[NM];
#pragma unroll 1
  for (int w = 0; w < NM; ++w) {
    uint32_t m = tie[w], a = 0u, e = 0u;
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      const int bit = 32 * w + b;
      const uint32_t full = float_to_ordered(mine[(bit >> 2) * TK_TILE + (bit & 3)]);
      a |= (full > T ? 1u : 0u) << b;
      e |= (full == T ? 1u : 0u) << b;
    }
    tgt[w] = a;
    teq[w] = e;
  }
  // class of position (j, c): bit 0 = key > T, bit 1 = key == T
#define CLS(j, c)                                                                             \
  (HI(j, c) > P16 ? 1u                                                                        \
                  : ((((tgt[(4 * (j) + (c)) >> 5] >> ((4 * (j) + (c)) & 31)) & 1u)) |            \
                     (((teq[(4 * (j) + (c)) >> 5] >> ((4 * (j) + (c)) & 31)) & 1u) << 1)))

  // counts (packed: > T in the low 16 bits, == T in the high 16 bits) per (tile, wave)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < tiles) {
      uint32_t pc = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t cl = CLS(j, c);
        pc += (cl & 1u) | ((cl >> 1) << 16);
      }
      const uint32_t incl = wave_incl_scan_packed(pc);
      if (lane == 63) {
        cnt[j * TK_WAVES + wave][0] = incl & 0xFFFFu;
        cnt[j * TK_WAVES + wave][1] = incl >> 16;
      }
    }
  }
  __syncthreads();
  // exclusive scan over the tiles*16 (tile, wave) totals, in position order
  const int ne = tiles * TK_WAVES;  // <= 512 <= 2 * TK_THREADS
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const uint32_t g0 = e0 < ne ? cnt[e0][0] : 0u, q0 = e0 < ne ? cnt[e0][1] : 0u;
  const uint32_t g1 = e1 < ne ? cnt[e1][0] : 0u, q1 = e1 < ne ? cnt[e1][1] : 0u;
  uint32_t eq_excl;
  const uint32_t gt_excl = block_excl_scan2(g0 + g1, q0 + q1, sw, eq_excl);
  __syncthreads();  // every thread has read cnt and sw
  if (e0 < ne) { cnt[e0][0] = gt_excl; cnt[e0][1] = eq_excl; }
  if (e1 < ne) { cnt[e1][0] = gt_excl + g0; cnt[e1][1] = eq_excl + q0; }
  __syncthreads();
  // selected before position p = (# keys > T before p) + min(# keys == T before p, need)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < tiles) {
      uint32_t cls[4], pc = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cls[c] = CLS(j, c);
        pc += (cls[c] & 1u) | ((cls[c] >> 1) << 16);
      }
      const uint32_t excl = wave_incl_scan_packed(pc) - pc;
      uint32_t gb = cnt[j * TK_WAVES + wave][0] + (excl & 0xFFFFu);
      uint32_t qb = cnt[j * TK_WAVES + wave][1] + (excl >> 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool gt = cls[c] == 1u, eq = cls[c] == 2u;
        const uint32_t at = gb + min(qb, need);
        if ((gt || (eq && qb < need)) && at < (uint32_t)k) out[at] = j * TK_TILE + 4 * tid + c;
        gb += gt;
        qb += eq;
      }
    }
  }
#undef CLS
#undef HI
}

size_t topk_workspace_bytes(const SeqInfo&, int) { return 0; }

hipError_t launch_topk(const SeqInfo& s, const float* scores, int64_t ld, int k, int32_t* idx,
                       void*, size_t, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int tiles = (s.max_n + TK_TILE - 1) / TK_TILE;
  const dim3 grid(s.T), block(TK_THREADS);
  if (tiles <= 2)
    hipLaunchKernelGGL(topk_reg_kernel<2>, grid, block, 0, st, s.B, s.cu_q, s.cu_k, scores, ld, k, idx);
  else if (tiles <= 8)
    hipLaunchKernelGGL(topk_reg_kernel<8>, grid, block, 0, st, s.B, s.cu_q, s.cu_k, scores, ld, k, idx);
  else if (tiles <= 32)
    hipLaunchKernelGGL(topk_reg_kernel<32>, grid, block, 0, st, s.B, s.cu_q, s.cu_k, scores, ld, k, idx);
  else
    hipLaunchKernelGGL(topk_row_kernel, grid, block, 0, st, s.B, s.cu_q, s.cu_k, scores, ld, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
