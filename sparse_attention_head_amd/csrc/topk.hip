// Causal per-row top-k selection on gfx950.
//
// For each query row: the min(k, pos+1) positions s <= pos with the largest index scores
// (page "A paper signed by Liang Wenfeng: The most powerful open-source Agent model of DeepSeek
// has made a big splash" (36kr), section "02. Built on the final version of DeepSeek-V3.1, DSA
// makes model computation smarter": retrieve only the entries with the top-k index scores; page
// "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models" (paper digest), section "Key
// claims", paper section 2.1, Eq. 2).
// Ties prefer the lower position, +0 equals -0, output ascending and padded with -1.
//
// Method (exact, deterministic): scores map to order-preserving 32-bit keys. A radix select over
// the key digits (at most 11 bits each, most significant first) finds the k-th largest key T and
// the number `need` of keys equal to T that belong to the selection; the output keeps every key > T
// and the `need` lowest positions with key == T, in ascending position order. Three kernels share
// these semantics: a streaming kernel that reads each row once and selects over a short list of
// candidates above a sampled floor (k <= 2048, rows up to 131072), a register-resident kernel for
// larger k, and a multi-pass kernel straight from global memory for longer rows (also the
// streaming kernel's fallback).
#include "dsa_internal.h"
#include "device_common.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

// Exact selection for one row straight from global memory with NTH threads: three histogram
// passes (key bits 31..21, 20..10, 9..0) find the k-th largest key T and how many keys equal to T
// are taken (`need`); then an ordered compaction in position order keeps every key > T and the
// first `need` keys == T. n > k. hist: 2048 words, xch: [2][NTH/64][2].
template <int NTH>
__device__ void topk_row_exact(const float* __restrict__ row, int n, int k, int32_t* __restrict__ out,
                               uint32_t* hist, uint32_t (*xch)[NTH / 64][2], uint32_t* s_digit,
                               uint32_t* s_above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)k;  // how many of the keys matching `prefix` still go in
  const int n4 = n & ~3;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += NTH) hist[i] = 0;
    __syncthreads();
    for (int i = tid * 4; i < n4; i += NTH * 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + i);
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = float_to_ordered(e[j]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
      }
    }
    for (int i = n4 + tid; i < n; i += NTH) {
      const uint32_t u = float_to_ordered(row[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    select_bin(hist, nb, need, s_digit, s_above);
    prefix |= *s_digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    need -= *s_above;
  }
  const uint32_t T = prefix;  // the k-th largest key; `need` >= 1 keys equal to T are taken

  // ordered compaction: selected before i = (# keys > T before i) + min(# keys == T before i, need)
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0, it = 0; base < n; base += NTH, ++it) {
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
    for (int v = 0; v < NTH / 64; ++v) {
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

__global__ void __launch_bounds__(TK_THREADS)
topk_row_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t xch[2][TK_WAVES][2];
  __shared__ uint32_t s_digit, s_above;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int n = L.pos + 1;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;

  if (n <= k) {  // every candidate is selected
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  topk_row_exact<TK_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
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

// Exclusive prefix sums of a and b over the workgroup in thread order (b's in excl_b): a
// data-parallel scan within each wave (lane moves, no LDS round trips), the wave totals through
// sw (2 words per wave), then lane i < wave reads wave i's totals and one more wave scan adds
// them up, so no thread walks the waves before it one by one. Begins the LDS exchange with a
// barrier; every thread of the workgroup must call it.
__device__ __forceinline__ uint32_t block_excl_scan2(uint32_t a, uint32_t b, uint32_t* sw,
                                                     uint32_t& excl_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) { sw[2 * wave] = xa; sw[2 * wave + 1] = xb; }
  __syncthreads();
  const uint32_t pa = wave_incl_scan(lane < wave ? sw[2 * lane] : 0u);
  const uint32_t pb = wave_incl_scan(lane < wave ? sw[2 * lane + 1] : 0u);
  const uint32_t ba = (uint32_t)__builtin_amdgcn_readlane((int)pa, 63);
  const uint32_t bb = (uint32_t)__builtin_amdgcn_readlane((int)pb, 63);
  excl_b = bb + xb - b;
  return ba + xa - a;
}

constexpr int TK_TILE = 4 * TK_THREADS;      // positions per tile (one float4 per thread)
constexpr int TK_CHUNK_TILES = 2;              // tiles per staged chunk (32 KB)
constexpr int TK_RING = 4;                     // staged chunks in flight


// Register-resident selection for rows of up to 4096 * NT candidates (one workgroup per row).
//  1. The row streams through LDS (4 chunks of 32 KB in flight, DMA) into registers: thread t
//     keeps the upper 16 bits of the keys of positions 4096j + 4t + c (c = 0..3), two per
//     register. The histogram of digit 1 (key bits 31..21) is built on the way: fully for the
//     first 8192 positions, and above a floor bin chosen from that sample for the rest (exact: if
//     fewer than k keys turn out to lie above the floor, the histogram is rebuilt from registers).
//  2. One pass over the registers marks each position "above" (digit 1 > d1) or "candidate"
//     (digit 1 == d1) in per-thread bitmasks.
//  3. The candidates -- the keys of one 11-bit bin, a small share of the row -- are refined by
//     re-reading their full keys: digits 2 (bits 20..16), 3 (15..8) and 4 (7..0), then their
//     class against the threshold T.
//  4. Ordered compaction from the bitmasks: per (tile, wave) counts from ballots, one block-wide
//     exclusive scan in (tile, wave) order -- which is position order -- and per-lane offsets
//     from lanes-below popcounts.
template <int NT>
__global__ void __launch_bounds__(TK_THREADS)
topk_reg_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx) {
  constexpr int NCH = (NT + TK_CHUNK_TILES - 1) / TK_CHUNK_TILES;  // staged chunks per row
  constexpr int NM = (4 * NT + 31) / 32;     // 32-bit words of per-thread position masks
  __shared__ __attribute__((aligned(16))) float stage[TK_RING][TK_CHUNK_TILES * TK_TILE];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t cnt[NT * TK_WAVES][2];  // per (tile, wave): keys > T, keys == T
  __shared__ uint32_t sw[2 * TK_WAVES];
  __shared__ uint32_t s_digit, s_above, s_floor;

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
  const int chunks = (tiles + TK_CHUNK_TILES - 1) / TK_CHUNK_TILES;
  for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;

  // Staging: chunk c (tiles 2c, 2c+1) is copied into stage[c % TK_RING] by 32 DMA instructions,
  // two per wave; lane l of instruction i of wave w copies the float4 at chunk offset
  // (2w + i)*256 + 4l. Float4s starting at or past the end of the row read the row start instead
  // (their values are discarded; a float4 straddling the end stays inside ld >= round_up(n, 4)).
  auto issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int off = (2 * wave + i) * 256;
      const int e = c * TK_CHUNK_TILES * TK_TILE + off + 4 * lane;
      const float* src = row + (e < n ? e : 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                       (__attribute__((address_space(3))) void*)(&stage[c % TK_RING][off]),
                                       16, 0, 0);
    }
  };
#pragma unroll
  for (int c = 0; c < TK_RING - 1; ++c)
    if (c < chunks) issue(c);

  uint32_t hk[2 * NT];
  uint32_t floor_bin = 0;
  __syncthreads();  // hist cleared
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c < chunks) {  // uniform
      if (c + TK_RING - 1 < chunks) {
        issue(c + TK_RING - 1);
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");  // chunk c has landed (3 newer in flight)
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < TK_CHUNK_TILES; ++h) {
        const int j = c * TK_CHUNK_TILES + h;
        if (j < NT) {
          const int e = j * TK_TILE + 4 * tid;
          const float4 v = *reinterpret_cast<const float4*>(&stage[c % TK_RING][h * TK_TILE + 4 * tid]);
          const float f[4] = {v.x, v.y, v.z, v.w};
          uint32_t k4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) k4[q] = e + q < n ? float_to_ordered(f[q]) : 0u;
          hk[2 * j] = (k4[0] >> 16) | (k4[1] & 0xFFFF0000u);
          hk[2 * j + 1] = (k4[2] >> 16) | (k4[3] & 0xFFFF0000u);
          asm volatile("" : "+v"(hk[2 * j]), "+v"(hk[2 * j + 1]));
          if (j < tiles)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t d = k4[q] >> 21;
              if (d >= floor_bin) atomicAdd(&hist[d], 1u);
            }
        }
      }
      if (c == 0 && chunks > 1) {
        // floor bin: from the first 8192 positions (a sample), the bin holding the
        // (4 k S / n + 64)-th largest key -- several times the expected share above the
        // threshold; later keys below it are not binned
        __syncthreads();
        const uint32_t want = (uint32_t)min((int64_t)TK_CHUNK_TILES * TK_TILE,
                                            4LL * k * (TK_CHUNK_TILES * TK_TILE) / n + 64);
        select_bin(hist, 2048, want, &s_digit, &s_above);
        if (tid == 0) s_floor = s_digit;
        __syncthreads();
        floor_bin = s_floor;
      }
      __syncthreads();  // stage[c % TK_RING] may be refilled
    } else {
#pragma unroll
      for (int h = 0; h < TK_CHUNK_TILES; ++h) {
        const int j = c * TK_CHUNK_TILES + h;
        if (j < NT) { hk[2 * j] = 0u; hk[2 * j + 1] = 0u; }
      }
    }
  }
#define HI(j, c) ((hk[2 * (j) + ((c) >> 1)] >> (16 * ((c) & 1))) & 0xFFFFu)

  uint32_t need = (uint32_t)k;
  // exact check of the floor: at least k keys must lie in bins >= floor_bin (only keys of the
  // first chunk were binned below it, and those bins are never reached in that case)
  if (tid == 0) s_digit = 0xFFFFFFFFu;
  __syncthreads();
  select_bin(hist, 2048, need, &s_digit, &s_above);
  if (s_digit == 0xFFFFFFFFu || s_digit < floor_bin) {  // uniform: rebuild from registers
    __syncthreads();
    for (int i = tid; i < 2048; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j)
      if (j < tiles)
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&hist[HI(j, c) >> 5], 1u);
    __syncthreads();
    select_bin(hist, 2048, need, &s_digit, &s_above);
  }
  const uint32_t d1 = s_digit;
  need -= s_above;

  // above / candidate bitmasks (bit 4j + c)
  uint32_t abv[NM], cand[NM];
#pragma unroll
  for (int w = 0; w < NM; ++w) { abv[w] = 0u; cand[w] = 0u; }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t d = HI(j, c) >> 5;
      abv[(4 * j + c) >> 5] |= (d > d1 ? 1u : 0u) << ((4 * j + c) & 31);
      cand[(4 * j + c) >> 5] |= (d == d1 ? 1u : 0u) << ((4 * j + c) & 31);
    }
  const float* mine = row + 4 * tid;  // position of bit b: (b / 4) * TK_TILE + 4 * tid + b % 4
  // The thread's first CK candidates: full keys loaded once into registers (independent loads,
  // in flight together). Threads with more candidates re-read the rest in each pass below.
  constexpr int CK = 4;
  uint32_t ckey[CK], cbit[CK];
  int ncand = 0;
  uint32_t rest[NM];  // candidates beyond the first CK
#pragma unroll
  for (int w = 0; w < NM; ++w) rest[w] = cand[w];
#pragma unroll
  for (int i = 0; i < CK; ++i) {
    cbit[i] = 0xFFFFFFFFu;
    ckey[i] = 0u;
#pragma unroll
    for (int w = 0; w < NM; ++w) {
      if (cbit[i] == 0xFFFFFFFFu && rest[w]) {
        const int b = __ffs(rest[w]) - 1;
        rest[w] &= rest[w] - 1;
        cbit[i] = 32 * w + b;
      }
    }
    if (cbit[i] != 0xFFFFFFFFu) {
      ckey[i] = float_to_ordered(mine[(cbit[i] >> 2) * TK_TILE + (cbit[i] & 3)]);
      ++ncand;
    }
  }
  uint32_t rest_or = 0u;
#pragma unroll
  for (int w = 0; w < NM; ++w) rest_or |= rest[w];
  const bool any_rest = __ballot(rest_or != 0u) != 0ull;  // uniform: rare

  // digits 2, 3, 4 over the candidates' full keys (key bits 20..16, 15..8, 7..0)
  uint32_t low_prefix = d1 << 21, low_mask = 0xFFE00000u;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 16 : (pass == 1 ? 8 : 0);
    const int nb = pass == 0 ? 32 : 256;
    __syncthreads();
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CK; ++i)
      if (i < ncand && (ckey[i] & low_mask) == low_prefix)
        atomicAdd(&hist[(ckey[i] >> shift) & (uint32_t)(nb - 1)], 1u);
    if (any_rest) {
#pragma unroll 1
      for (int w = 0; w < NM; ++w) {
        uint32_t m = rest[w];
        while (m) {
          const int bit = 32 * w + __ffs(m) - 1;
          m &= m - 1;
          const uint32_t key = float_to_ordered(mine[(bit >> 2) * TK_TILE + (bit & 3)]);
          if ((key & low_mask) == low_prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
    }
    __syncthreads();
    select_bin(hist, nb, need, &s_digit, &s_above);
    low_prefix |= s_digit << shift;
    low_mask |= (uint32_t)(nb - 1) << shift;
    need -= s_above;
  }
  const uint32_t T = low_prefix;  // the k-th largest key; `need` keys == T go in

  // final classes: gt = above, or a candidate whose key > T; eq = a candidate whose key == T
  uint32_t gtm[NM], eqm[NM];
  uint32_t any_eq_lane = 0u;
#pragma unroll
  for (int w = 0; w < NM; ++w) {
    uint32_t a = 0u, e = 0u;
#pragma unroll
    for (int i = 0; i < CK; ++i)
      if (i < ncand && (int)(cbit[i] >> 5) == w) {
        a |= (ckey[i] > T ? 1u : 0u) << (cbit[i] & 31);
        e |= (ckey[i] == T ? 1u : 0u) << (cbit[i] & 31);
      }
    gtm[w] = a;
    eqm[w] = e;
  }
  if (any_rest) {
#pragma unroll 1
    for (int w = 0; w < NM; ++w) {
      uint32_t m = rest[w], a = 0u, e = 0u;
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        const int bit = 32 * w + b;
        const uint32_t key = float_to_ordered(mine[(bit >> 2) * TK_TILE + (bit & 3)]);
        a |= (key > T ? 1u : 0u) << b;
        e |= (key == T ? 1u : 0u) << b;
      }
      // runtime word index: merge through a compile-time loop (keeps the arrays in registers)
#pragma unroll
      for (int v = 0; v < NM; ++v)
        if (v == w) { gtm[v] |= a; eqm[v] |= e; }
    }
  }
#pragma unroll
  for (int w = 0; w < NM; ++w) {
    any_eq_lane |= eqm[w];
    gtm[w] |= abv[w];
  }
  const bool any_eq = __ballot(any_eq_lane != 0u) != 0ull;  // uniform

  // counts per (tile, wave) from ballots
#define NIB(msk, j) (((msk)[(j) >> 3] >> (4 * ((j) & 7))) & 15u)
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < tiles) {
      const uint32_t g4 = NIB(gtm, j);
      uint32_t ng = 0u, nq = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) ng += (uint32_t)__popcll(__ballot((g4 >> c) & 1u));
      if (any_eq) {
        const uint32_t q4 = NIB(eqm, j);
#pragma unroll
        for (int c = 0; c < 4; ++c) nq += (uint32_t)__popcll(__ballot((q4 >> c) & 1u));
      }
      if (lane == 0) {
        cnt[j * TK_WAVES + wave][0] = ng;
        cnt[j * TK_WAVES + wave][1] = nq;
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
      const uint32_t gt4 = NIB(gtm, j), eq4 = any_eq ? NIB(eqm, j) : 0u;
      if (__ballot((gt4 | eq4) != 0u)) {  // uniform: skip tiles with nothing selected in this wave
        uint32_t gb = cnt[j * TK_WAVES + wave][0], qb = cnt[j * TK_WAVES + wave][1];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          gb += lanes_below_count(__ballot((gt4 >> c) & 1u));
          if (any_eq) qb += lanes_below_count(__ballot((eq4 >> c) & 1u));
        }
        uint32_t m = gt4 | eq4;
        while (m) {  // the lane's few selected positions of this tile, in position order
          const int c = __ffs(m) - 1;
          m &= m - 1;
          const uint32_t below = (1u << c) - 1u;
          const uint32_t g_at = gb + (uint32_t)__popc(gt4 & below);
          const uint32_t q_at = qb + (uint32_t)__popc(eq4 & below);
          const bool take = ((gt4 >> c) & 1u) || q_at < need;
          const uint32_t at = g_at + min(q_at, need);
          if (take && at < (uint32_t)k) out[at] = j * TK_TILE + 4 * tid + c;
        }
      }
    }
  }
#undef NIB
#undef HI
}

// ------------------------------------------------------------------------------------------
// Streaming variant for k <= 2048 and rows of up to 131072 candidates (any batch size): one pass
// over the row with about two vector instructions per score, so that the pass runs at memory
// speed, and workgroups of sixteen waves with 76 KB of LDS, two per compute unit (the full 32
// waves), so that the selection work of one row overlaps the streaming of another and the
// latency-bound selection phases run on more threads.
//  0. Rows of at most 8192 positions are read into LDS whole and selected there directly: three
//     radix digits give the k-th largest key, then steps 5 and 6 below run on that copy.
//  1. Longer rows: a sample of 8 evenly spaced runs of 256, 512 or 1024 positions (about n/16 in
//     all) is kept in LDS; two radix digits (22 key bits) locate its `want`-th largest key and the
//     floor F is that 22-bit bin's lower edge; want = 1.3 k S / n aims at about 1.3 k keys (3
//     sigma above k and about 4 sigma below the list's capacity for independent scores).
//  2. The stream works on groups of 4 consecutive scores (one float4 per lane): a group whose
//     maximum reaches F is appended whole, with its position, to a list in LDS (structure of
//     arrays). Per batch of 4 groups per lane one atomic per wave reserves the slots; each lane
//     then stores every group unconditionally, to its slot or, without a hit, to a spare slot of
//     its own, so the loop has no per-group branch.
//  3. The groups are compacted into a list of single keys >= F with their positions.
//  4. If there are more groups than slots, fewer than k or more than 4096 keys, or more than 2048
//     keys tie at the threshold, the row is redone exactly from global memory.
//  5. Radix select over the list: the k-th largest key T and how many keys equal to T are taken
//     (`need`, the lowest positions first; when fewer than all, a radix select over the tied
//     positions finds the last one taken). The digits start at the highest bit where F and the
//     list's largest key differ (every listed key lies between them).
//  6. The selected positions are marked in a bitmap; each thread owns a run of its words, one
//     block-wide exclusive scan of their popcounts gives the output offsets, and every thread
//     writes its positions in ascending order.
constexpr int TS_THREADS = 1024;
constexpr int TS_WAVES = TS_THREADS / 64;
constexpr int TS_MAXN = 131072;            // positions covered by the bitmap
constexpr int TS_MAXK = 2048;
constexpr int TS_GCAP = 3392;              // group slots
constexpr int TS_GSTRIDE = TS_GCAP + 64;   // words per group array: the slots, then one spare per lane
static_assert(TS_GSTRIDE % 64 == 0, "group arrays are 256-byte aligned (paired-store offsets)");
constexpr int TS_HCAP = 4096;              // keys in the compacted list
constexpr int TS_SEG = 1024;               // positions per sample run, at most
constexpr int TS_SEGS = 8;
constexpr int TS_SAMPLE = TS_SEG * TS_SEGS;   // 8192
constexpr int TS_MAXEQ = 2048;             // tied keys handled in LDS
constexpr int TS_REGION = 5 * TS_GSTRIDE;  // sample | group arrays x, y, z, w, position | keys, positions, bitmap
static_assert(TS_SAMPLE <= TS_REGION, "the sample shares the region");
static_assert(2 * TS_HCAP + TS_MAXN / 32 <= TS_REGION, "compacted list and bitmap share the region");
constexpr int TS_UNROLL = 4;               // float4 loads per thread and batch (two batches in flight)
constexpr int TS_UNROLL_PF = 8;            // the same with one workgroup per compute unit (PF launches)
constexpr int TS_GPT = (TS_GCAP + TS_THREADS - 1) / TS_THREADS;   // groups per thread in the compaction

// Largest of the four values (finite inputs: no NaN handling, which fmaxf would add per operand).
__device__ __forceinline__ float max4(float4 v) {
  float t, r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(t) : "v"(v.x), "v"(v.y), "v"(v.z));
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(t), "v"(v.w));
  return r;
}

// The bin holding the need-th largest of the counted keys (nb bins, a power of two <= 2048;
// counts from the top bin down), found by the whole workgroup of TS_THREADS: thread t owns the run
// of nb / TS_THREADS bins (at least one; threads past nb own none) that starts t runs below the
// top, so the keys above a thread's run are an exclusive prefix sum in thread order: a scan within
// each wave plus the totals of the waves before it (wsum, TS_WAVES words). The thread whose run
// holds the need-th key walks its bins and writes *s_digit and *s_above (keys in higher bins).
// Every thread then clears the bins it owns, so the histogram is zero again when the call
// returns. Called by all threads; ends with a barrier.
__device__ __forceinline__ void select_bin_block(uint32_t* hist, int nb, uint32_t need, uint32_t* wsum,
                                                 uint32_t* s_digit, uint32_t* s_above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = nb >= TS_THREADS ? nb / TS_THREADS : 1;   // 1 or 2
  const int b_hi = nb - 1 - tid * per;                      // the run's top bin (b_hi - per < b <= b_hi)
  uint32_t h0 = 0, h1 = 0;
  if (b_hi >= 0) {
    h0 = hist[b_hi];
    if (per == 2) h1 = hist[b_hi - 1];
  }
  const uint32_t sum = h0 + h1;
  const uint32_t incl = wave_incl_scan(sum);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  // totals of the waves before this one: lane i < wave reads wave i's, one sum across the lanes
  const uint32_t before = wave_incl_scan(lane < wave ? wsum[lane] : 0u);
  const uint32_t above = incl - sum + (uint32_t)__builtin_amdgcn_readlane((int)before, 63);
  if (b_hi >= 0) {
    if (above < need && above + h0 >= need) {
      *s_digit = (uint32_t)b_hi;
      *s_above = above;
    } else if (per == 2 && above + h0 < need && above + sum >= need) {
      *s_digit = (uint32_t)(b_hi - 1);
      *s_above = above + h0;
    }
    hist[b_hi] = 0;
    if (per == 2) hist[b_hi - 1] = 0;
  }
  __syncthreads();
}

// Radix select over `count` keys in LDS that all share `prefix` on the bits of `pmask`: digits of
// at most 11 bits resolve key bits hi..lo, most significant first. Returns the key prefix of the
// want-th largest key (bits below lo zero; the key itself when lo = 0) and how many of the keys
// with that prefix rank within the first `want` (*need_out). hist: 2048 words; wsum: TS_WAVES
// words. The histogram is cleared once; each pass's bin search leaves it zero for the next (whose
// digit is never wider).
__device__ __forceinline__ uint32_t lds_select(const uint32_t* keys, uint32_t count, uint32_t want,
                                               int hi, int lo, uint32_t prefix, uint32_t pmask,
                                               uint32_t* hist, uint32_t* wsum, uint32_t* s_digit,
                                               uint32_t* s_above, uint32_t* need_out) {
  const int tid = threadIdx.x;
  uint32_t need = want;
  if (hi >= lo) {
    const int nb0 = 1 << min(11, hi - lo + 1);
    for (int i = tid; i < nb0; i += TS_THREADS) hist[i] = 0;
    __syncthreads();
  }
#pragma unroll 1
  for (int top = hi; top >= lo;) {
    const int width = min(11, top - lo + 1);
    const int shift = top + 1 - width;
    const int nb = 1 << width;
    for (uint32_t c = tid; c < count; c += TS_THREADS) {
      const uint32_t u = keys[c];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    select_bin_block(hist, nb, need, wsum, s_digit, s_above);
    prefix |= *s_digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    need -= *s_above;
    top = shift - 1;
  }
  *need_out = need;
  return prefix;
}

// Largest value over the wave (prefix maximum with the same data-parallel steps as
// wave_incl_scan, read from the last lane).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// Marks the selection among `total` listed keys (ckey, positions cpos < 32 nw, or the list index
// when cpos is NULL: a whole row) -- every key above
// T and the `need` lowest positions among the keys equal to T -- in the row's bitmap (nw words,
// cleared by the caller), then writes the marked positions in ascending order to out[0..).
// Returns false (uniform, with nothing written to out) if more than TS_MAXEQ keys equal T; the
// caller then selects the row exactly instead. hist holds the tied positions (>= TS_MAXEQ
// words), scratch the tie select's histogram (2048 words; the key list may serve), *s_eq is zero
// on entry. Called by every thread; begins with a barrier.
__device__ __forceinline__ bool mark_and_emit(const uint32_t* ckey, const uint32_t* cpos, uint32_t total, uint32_t T,
                              uint32_t need, int nw, uint32_t* bmap, uint32_t* hist, uint32_t* scratch,
                              uint32_t* s_eq, uint32_t* s_digit, uint32_t* s_above, uint32_t* xch1,
                              int32_t* out) {
  const int tid = threadIdx.x;
  __syncthreads();   // the histogram space is reused for the tied positions
  for (uint32_t c = tid; c < total; c += TS_THREADS) {
    const uint32_t u = ckey[c], p = cpos ? cpos[c] : c;
    if (u > T) {
      atomicOr(&bmap[p >> 5], 1u << (p & 31));
    } else if (u == T) {
      const uint32_t e = atomicAdd(s_eq, 1u);
      if (e < (uint32_t)TS_MAXEQ) hist[e] = ~p;   // inverted: the largest are the lowest positions
    }
  }
  __syncthreads();
  const uint32_t eqc = *s_eq;
  if (eqc > (uint32_t)TS_MAXEQ) return false;
  // the tied keys taken are the `need` lowest positions: ~pos >= the need-th largest ~pos
  uint32_t cut = 0u;
  if (eqc > need) {
    uint32_t unused;
    cut = lds_select(hist, eqc, need, 31, 0, 0u, 0u, scratch, xch1, s_digit, s_above, &unused);
  }
  for (uint32_t e = tid; e < eqc; e += TS_THREADS) {
    const uint32_t ip = hist[e];
    if (ip >= cut) {
      const uint32_t p = ~ip;
      atomicOr(&bmap[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  // one scan over the bitmap, ascending output
  const int per = (nw + TS_THREADS - 1) / TS_THREADS;
  const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(bmap[w]);
  uint32_t unused3;
  uint32_t slot = block_excl_scan2(cnt, 0u, xch1, unused3);
  for (int w = w0; w < w1; ++w) {
    uint32_t sel = bmap[w];
    while (sel) {
      out[slot++] = w * 32 + (__ffs(sel) - 1);
      sel &= sel - 1;
    }
  }
  return true;
}

// At most 64 scalar registers: with the 83 the compiler otherwise takes, the hardware placed one
// workgroup per compute unit instead of two (measured: per-workgroup CU ids and timestamps), and
// the 128K-chunk selection took 586 instead of 454 us.
// PF (batches of at most one row per compute unit, where the kernel's register count no longer
// decides its residency): the first two stream batches are requested right after the sample, so
// their latency hides behind the floor select.
template <bool PF>
__global__ void __launch_bounds__(TS_THREADS) __attribute__((amdgpu_num_sgpr(64)))
topk_stream_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                   const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[2048];          // histograms; tied positions at the end
  __shared__ __attribute__((aligned(16))) uint32_t region[TS_REGION];
  __shared__ uint32_t xch[2][TS_WAVES][2];
  __shared__ uint32_t s_digit, s_above, s_count, s_eq, s_max;
  uint32_t* const ckey = region;
  uint32_t* const cpos = region + TS_HCAP;
  uint32_t* const bmap = region + 2 * TS_HCAP;

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int n = L.pos + 1;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;

  if (n <= k) {
    for (int i = tid; i < k; i += TS_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const int nw = (n + 31) >> 5;
  const int n4 = n & ~3;
  // batches of UNR float4 per lane, double-buffered (two register sets used in turn): the next
  // batch is in flight while the current one is scanned. PF launches (one workgroup per compute
  // unit, so registers to spare) take batches twice as large: there a long row's stream is bound
  // by the bytes one compute unit keeps in flight. Buffer loads: one resource per batch (starting
  // at the batch, covering the whole groups left in the row) and fixed lane offsets, so no
  // per-load address arithmetic; groups past the end read as zero (scan_batch then sets them to
  // -inf), so every batch issues the same UNR loads.
  constexpr int UNR = PF ? TS_UNROLL_PF : TS_UNROLL;
  constexpr int BATCH = TS_THREADS * 4 * UNR;
  auto load_batch = [&](int base, float4 (&v)[UNR]) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row) + base, (short)0, max(n4 - base, 0) * 4, 0x00020000);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, (u * TS_THREADS + tid) * 16, 0, 0);
      v[u] = make_float4(__uint_as_float(t[0]), __uint_as_float(t[1]), __uint_as_float(t[2]), __uint_as_float(t[3]));
    }
  };
  float4 va[UNR], vb[UNR];

  // 1. sample and floor
  const bool whole = n <= TS_SAMPLE;
  // a sample of about n/16 positions (2048 .. 8192) in 8 evenly spaced runs: the floor's target
  // rank in it (~166 at k = 2048) stays the same for every row length
  const int seg = n >= 12 * TS_SAMPLE ? TS_SEG : n >= 6 * TS_SAMPLE ? TS_SEG / 2 : TS_SEG / 4;
  const int S = whole ? n : TS_SEGS * seg;
  if (whole) {
    for (int i = tid; i < n; i += TS_THREADS) region[i] = float_to_ordered(row[i]);
  } else {
    // every sample load is issued before the first one is used; the PF batches after them, so
    // the sample arrives first and the batches stream in during the floor select
    float sv[TS_SAMPLE / TS_THREADS];
#pragma unroll
    for (int u = 0; u < TS_SAMPLE / TS_THREADS; ++u) {
      const int i = tid + u * TS_THREADS;
      if (i < S) {
        const int j = i / seg, o = i - j * seg;
        const int start = (int)((int64_t)j * (n - seg) / (TS_SEGS - 1));
        sv[u] = row[start + o];
      }
    }
    if constexpr (PF) {
      load_batch(0, va);
      load_batch(BATCH, vb);
    }
#pragma unroll
    for (int u = 0; u < TS_SAMPLE / TS_THREADS; ++u) {
      const int i = tid + u * TS_THREADS;
      if (i < S) region[i] = float_to_ordered(sv[u]);
    }
  }
  if (tid == 0) {
    s_count = 0;
    s_eq = 0;
    s_max = 0;
  }
  __syncthreads();
  if (whole) {
    // the whole row is in LDS: select the k-th largest key exactly (three digits), mark and write
    // straight from this copy (region[n..) and the bitmap past 2 TS_HCAP words do not overlap)
    for (int i = tid; i < nw; i += TS_THREADS) region[2 * TS_HCAP + i] = 0;
    uint32_t need;   // (lds_select starts with a barrier)
    const uint32_t T = lds_select(region, (uint32_t)n, (uint32_t)k, 31, 0, 0u, 0u, hist, &xch[0][0][0], &s_digit, &s_above,
                                  &need);
    if (!mark_and_emit(region, nullptr, (uint32_t)n, T, need, nw, region + 2 * TS_HCAP, hist, region, &s_eq,
                       &s_digit, &s_above, &xch[1][0][0], out))
      topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
    return;
  }
  static_assert(TS_SAMPLE <= 2 * TS_HCAP, "a whole-row sample stays below the bitmap");
  const uint32_t want = (uint32_t)max<int64_t>(1, min<int64_t>(S, (13 * (int64_t)k * S + 10 * (int64_t)n - 1) / (10 * (int64_t)n)));
  uint32_t unused;
  const uint32_t F = lds_select(region, (uint32_t)S, want, 31, 10, 0u, 0u, hist, &xch[0][0][0], &s_digit, &s_above,
                                &unused);
  __syncthreads();   // every thread has F before the group arrays overwrite the sample

  // 2. stream. Scores are compared as floats: the order-preserving key map is monotone and folds
  // -0 onto +0, which the float comparison treats as equal too.
  const float Ff = __uint_as_float((F & 0x80000000u) ? (F & 0x7FFFFFFFu) : ~F);
  // group arrays; a lane's slot address is its word index * 4, the arrays follow at multiples of
  // TS_GSTRIDE words
  const uint32_t spare4 = 4u * (uint32_t)(TS_GCAP + lane);
  auto store_group = [&](uint32_t slot4, float4 v, uint32_t p) {   // slot4 = 4 * slot
    uint32_t* a = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(region) + slot4);
    a[0] = __float_as_uint(v.x);
    a[TS_GSTRIDE] = __float_as_uint(v.y);
    a[2 * TS_GSTRIDE] = __float_as_uint(v.z);
    a[3 * TS_GSTRIDE] = __float_as_uint(v.w);
    a[4 * TS_GSTRIDE] = p;
  };
  auto scan_batch = [&](int base, float4 (&v)[UNR]) {
    if (base + BATCH > n4) {   // uniform: the partial batch
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (base + (u * TS_THREADS + tid) * 4 >= n4) v[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    bool sel[UNR];      // group u reaches F
    uint64_t m[UNR];    // wave-uniform: the lanes where it does
    uint32_t hits = 0;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      sel[u] = max4(v[u]) >= Ff;
      m[u] = __ballot(sel[u]);
      hits += (uint32_t)__popcll(m[u]);
    }
    if (hits) {   // uniform
      uint32_t wbase = 0;
      if (lane == 0) wbase = atomicAdd(&s_count, hits);
      uint32_t run = __builtin_amdgcn_readfirstlane(wbase);
      if (run + hits <= (uint32_t)TS_GCAP) {   // uniform; on overflow the row is redone exactly
        const uint32_t p0 = (uint32_t)(base + tid * 4);
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const uint32_t at4 = 4u * lanes_below_count(m[u]) + 4u * run;
          store_group(sel[u] ? at4 : spare4, v[u], p0 + (uint32_t)(u * TS_THREADS * 4));
          run += (uint32_t)__popcll(m[u]);
        }
      }
    }
  };
  const int nb = (n4 + BATCH - 1) / BATCH;
  if (nb > 0) {   // n4 >= 4
    if constexpr (!PF) load_batch(0, va);
    for (int j = 0;;) {
      if (!PF || j > 0) load_batch((j + 1) * BATCH, vb);   // (PF: batch 1 is already in flight)
      scan_batch(j * BATCH, va);
      if (++j >= nb) break;
      load_batch((j + 1) * BATCH, va);
      scan_batch(j * BATCH, vb);
      if (++j >= nb) break;
    }
  }
  if (tid == 0 && n4 < n) {   // the last, partial group
    const float4 t = *reinterpret_cast<const float4*>(row + n4);   // inside the row: ld >= round_up(n, 4)
    const float4 v = make_float4(t.x, n4 + 1 < n ? t.y : -INFINITY, n4 + 2 < n ? t.z : -INFINITY, -INFINITY);
    if (max4(v) >= Ff) {
      const uint32_t at = atomicAdd(&s_count, 1u);
      if (at < (uint32_t)TS_GCAP) store_group(4u * at, v, (uint32_t)n4);
    }
  }
  __syncthreads();

  // 3. compaction of the groups into single keys >= F (order does not matter)
  const uint32_t groups = s_count;
  if (groups > (uint32_t)TS_GCAP) {
    topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
    return;
  }
  float4 gv[TS_GPT];
  uint32_t gp[TS_GPT], mine = 0;
#pragma unroll
  for (int j = 0; j < TS_GPT; ++j) {
    const uint32_t g = (uint32_t)(tid + j * TS_THREADS);
    if (g < groups) {
      gv[j] = make_float4(__uint_as_float(region[g]), __uint_as_float(region[TS_GSTRIDE + g]),
                          __uint_as_float(region[2 * TS_GSTRIDE + g]), __uint_as_float(region[3 * TS_GSTRIDE + g]));
      gp[j] = region[4 * TS_GSTRIDE + g];
    } else {
      gv[j] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      gp[j] = 0;
    }
    mine += (gv[j].x >= Ff) + (gv[j].y >= Ff) + (gv[j].z >= Ff) + (gv[j].w >= Ff);
  }
  uint32_t unused_b;
  uint32_t at = block_excl_scan2(mine, 0u, &xch[0][0][0], unused_b);   // barrier: all groups read
  uint32_t total = 0;
  for (int w = 0; w < TS_WAVES; ++w) total += xch[0][w][0];
  if (total < (uint32_t)k || total > (uint32_t)TS_HCAP) {
    __syncthreads();   // the fallback reuses xch
    topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
    return;
  }
  uint32_t kmax = 0u;   // largest key of the thread's hits (ordered keys are >= 0)
#pragma unroll
  for (int j = 0; j < TS_GPT; ++j) {
    const float e[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (e[c] >= Ff) {
        const uint32_t u = float_to_ordered(e[c]);
        ckey[at] = u;
        cpos[at] = gp[j] + (uint32_t)c;
        kmax = max(kmax, u);
        ++at;
      }
  }
  kmax = wave_max(kmax);
  if (lane == 0) atomicMax(&s_max, kmax);
  for (int i = tid; i < nw; i += TS_THREADS) bmap[i] = 0;
  __syncthreads();

  // 5. radix select over the list; keys above T go to the bitmap, tied positions to a list
  uint32_t need;
  // every key lies in [F, M]: the bits above the highest one where F and M differ are common, and
  // the digits start below them
  const uint32_t M = s_max;
  const int h = (M == F) ? -1 : 31 - __clz(M ^ F);
  // the bits above h (all bits for h = -1, none for h = 31), as one 64-bit shift: a select between
  // all-ones and the 32-bit form was merged by the compiler into a test of the shifted value, which
  // is zero for h = 31 as for h = -1, and gave all-ones for h = 31 (a floor below zero with a
  // maximum above it)
  const uint32_t common = (uint32_t)(~0ull << (h + 1));
  const uint32_t T = lds_select(ckey, total, (uint32_t)k, h, 0, F & common, common, hist, &xch[0][0][0], &s_digit,
                                &s_above, &need);
  // 6. marking and ascending output
  if (!mark_and_emit(ckey, cpos, total, T, need, nw, bmap, hist, ckey, &s_eq, &s_digit, &s_above,
                     &xch[1][0][0], out))
    topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
}

// ------------------------------------------------------------------------------------------
// Merge of the fused decode top-k. The decode indexer kept, for every chunk of kDecodeChunk keys
// of a row, every key at or above a cut (all of them when the chunk is short), with the count,
// the cut and flags in the chunk's metadata. One workgroup per row gathers the kept keys, finds
// the k-th largest T among them and `need` as the streaming kernel does, and checks that no chunk
// dropped a key that could rank: every chunk that dropped keys must have its cut at or below T
// (its dropped keys are then below T, so the kept keys contain every key above T and every key
// equal to T). If that fails, a chunk overflowed, or the kept keys do not fit in LDS, the row is
// selected exactly from its scores instead.
constexpr int TM_HCAP = 12288;                        // kept keys of a row held in LDS
constexpr int TM_MAXCH = TS_MAXN / kDecodeChunk;      // chunks of a row (128)

__global__ void __launch_bounds__(TS_THREADS)
topk_merge_decode_kernel(int B, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                         const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx,
                         DecodeCand cand) {
  __shared__ uint32_t hist[2048];
  __shared__ __attribute__((aligned(16))) uint32_t ckey[TM_HCAP];
  __shared__ uint32_t cpos[TM_HCAP];
  __shared__ uint32_t bmap[TS_MAXN / 32];
  __shared__ uint32_t c_off[TM_MAXCH], c_cnt[TM_MAXCH];
  __shared__ uint32_t xch[2][TS_WAVES][2];
  __shared__ uint32_t s_digit, s_above, s_eq, s_bad;
  static_assert(TM_HCAP >= 2048, "the key list doubles as the tie select's histogram");

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RowLoc L = locate_row(cu_q, cu_k, B, r);
  const int n = L.pos + 1;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores + (int64_t)r * ld;
  if (n <= k) {
    for (int i = tid; i < k; i += TS_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const int nch = (n + kDecodeChunk - 1) / kDecodeChunk;   // <= TM_MAXCH (n <= TS_MAXN)
  const uint32_t* meta = cand.meta + (int64_t)r * cand.nch * 4;
  uint32_t cnt = 0, over = 0;
  if (tid < nch) {
    cnt = meta[4 * tid];
    over = (meta[4 * tid + 2] >> 1) & 1u;
  }
  uint32_t unused;
  const uint32_t off = block_excl_scan2(cnt, over, &xch[0][0][0], unused);
  uint32_t total = 0, overflow = 0;
  for (int w = 0; w < TS_WAVES; ++w) {
    total += xch[0][w][0];
    overflow += xch[0][w][1];
  }
  if (overflow || total > (uint32_t)TM_HCAP || total < (uint32_t)k) {   // uniform
    __syncthreads();   // the fallback reuses xch
    topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
    return;
  }
  if (tid < nch) {
    c_off[tid] = off;
    c_cnt[tid] = cnt;
  }
  const int nw = (n + 31) >> 5;
  for (int i = tid; i < nw; i += TS_THREADS) bmap[i] = 0;
  if (tid == 0) {
    s_eq = 0;
    s_bad = 0;
  }
  __syncthreads();
  // gather: wave w copies the kept keys of chunks w, w + 16, ...
  for (int ch = wave; ch < nch; ch += TS_WAVES) {
    const int64_t src = ((int64_t)r * cand.nch + ch) * cand.stride;
    const uint32_t o = c_off[ch], cc = c_cnt[ch];
    for (uint32_t j = lane; j < cc; j += 64) {
      ckey[o + j] = cand.key[src + j];
      cpos[o + j] = cand.pos[src + j];
    }
  }
  // (lds_select starts with a barrier)
  uint32_t need;
  const uint32_t T = lds_select(ckey, total, (uint32_t)k, 31, 0, 0u, 0u, hist, &xch[0][0][0], &s_digit, &s_above,
                                &need);
  if (tid < nch && (meta[4 * tid + 2] & 1u) == 0 && meta[4 * tid + 1] > T) s_bad = 1;
  __syncthreads();
  if (s_bad || !mark_and_emit(ckey, cpos, total, T, need, nw, bmap, hist, ckey, &s_eq, &s_digit, &s_above,
                              &xch[1][0][0], out))
    topk_row_exact<TS_THREADS>(row, n, k, out, hist, xch, &s_digit, &s_above);
}

hipError_t launch_topk_merge_decode(const SeqInfo& s, const float* scores, int64_t ld, int k,
                                    int32_t* idx, const DecodeCand& cand, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_merge_decode_kernel, dim3(s.T), dim3(TS_THREADS), 0, st, s.B, s.cu_q, s.cu_k,
                     scores, ld, k, idx, cand);
  return hipGetLastError();
}

size_t topk_workspace_bytes(const SeqInfo&, int) { return 0; }

hipError_t launch_topk(const SeqInfo& s, const float* scores, int64_t ld, int k, int32_t* idx,
                       void*, size_t, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int tiles = (s.max_n + TK_TILE - 1) / TK_TILE;
  const dim3 grid(s.T), block(TK_THREADS);
  // the streaming kernel for k <= 2048 and rows up to 131072 candidates, large batches and decode
  // alike (it also finishes a lone row sooner than the register-resident kernel); the others for
  // larger k and longer rows
  if (k <= TS_MAXK && s.max_n <= TS_MAXN)
  {
    if (s.T <= kTargetCUs)
      hipLaunchKernelGGL(topk_stream_kernel<true>, grid, dim3(TS_THREADS), 0, st, s.B, s.cu_q, s.cu_k, scores,
                         ld, k, idx);
    else
      hipLaunchKernelGGL(topk_stream_kernel<false>, grid, dim3(TS_THREADS), 0, st, s.B, s.cu_q, s.cu_k, scores,
                         ld, k, idx);
  }
  else if (tiles <= 2)
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
