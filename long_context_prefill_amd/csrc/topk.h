// Exact block-wide top-k with ties broken towards the lowest index.
//
// Selection order: score descending, then index ascending.  The k-th largest
// key is found by an MSB-first radix select on order-preserving 32-bit keys
// (4 passes of 8 bits, integer histograms, so the result is unique and
// run-to-run identical); then every element above it, plus the lowest-indexed
// elements equal to it, are written out in ascending index order by an
// ordered (stable) compaction.
#pragma once

#include "common.h"

namespace minf {

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan over the NT threads of a block; *total gets the sum.
// `sh` needs NT/64 + 1 ints.
template <int NT>
__device__ __forceinline__ int block_scan_excl(int x, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = x;
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) { const int t = sh[w]; sh[w] = run; run += t; }
    sh[NT / 64] = run;
  }
  __syncthreads();
  const int res = sh[wave] + v - x;
  *total = sh[NT / 64];
  __syncthreads();
  return res;
}

// Digit whose bin holds the rem-th largest key: bins are scanned from the top
// (digit 255 down), tot[d] is the bin count of digit d, held by thread d of
// the first four waves.  Returns (digit, rank of the element within the bin)
// to thread 0 through sh.
__device__ __forceinline__ void pick_digit(int tot, int rem, uint32_t prefix, uint32_t mask, int shift, int* scan,
                                           uint32_t* out_prefix, uint32_t* out_mask, int* out_rem) {
  // inclusive sum of tot over digits >= d (reverse scan over 256 threads)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int v = tid < 256 ? tot : 0;
  // within the wave: sum over lanes >= lane
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_down(v, off);
    if (lane + off < 64) v += y;
  }
  if (lane == 0 && wave < 4) scan[wave] = v;
  __syncthreads();
  if (tid < 256) {
    int above = 0;
    for (int w = wave + 1; w < 4; ++w) above += scan[w];
    const int incl = v + above;          // keys with digit >= tid
    const int excl = incl - tot;          // keys with digit >  tid
    if (excl < rem && incl >= rem) {
      *out_prefix = prefix | ((uint32_t)tid << shift);
      *out_mask = mask | (0xffu << shift);
      *out_rem = rem - excl;
    }
  }
  __syncthreads();
}

// Adds one to hist[bin] for every lane with act set.  The keys of one row
// tend to share their top bytes, so most lanes of a wave fall into one or
// two bins, and plain atomics would queue on those counters: the lanes of
// the first two distinct bins (in lane order) are counted with one atomic
// each, the remaining lanes add their own one.
__device__ __forceinline__ void hist_add(int* hist, bool act, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  uint64_t am = __ballot(act);
  #pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (am == 0) return;
    const int lead = __ffsll((unsigned long long)am) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, lead);
    const uint64_t m = __ballot(act && bin == lb);
    if (lane == lead) atomicAdd(&hist[lb], __popcll(m));
    if ((m >> lane) & 1ull) act = false;
    am &= ~m;
  }
  if (act) atomicAdd(&hist[bin], 1);
}

// block_topk_reg selects the top min(k, n) of get(0..n-1), up to NT * E
// elements held in registers, and writes idx of their positions, ascending,
// to out[0..); out[min(k,n) .. cap) is filled with -1 (idx is the identity
// unless given).  Thread t reads elements [t*E, t*E + E) once;
// the four radix passes and the ordered compaction work on those registers.
// `get(i)` is called once for every i < NT * E (also past n, where its value
// is discarded), must be safe to call there and must not return NaN.  Slots past
// n hold key 0, below the key of every other float (-inf has key
// 0x007fffff): they can only fall into the lowest bin of a pass whose prefix
// is all zero, below every real key, so the k <= n largest keys, the
// threshold and the selection do not depend on them and no pass tests for
// them.
struct TopkRegShared {
  int hist[4][256];
  int scan[17];
  uint32_t prefix, mask;
  int remaining;
};

// The selection itself on keys already in registers: thread t holds the
// keys of elements lo .. lo + E - 1 (lo = t * E), key 0 for slots past n, and
// 0 < k < n.  The indices written are idx(element).
template <int NT, int E, typename Idx>
__device__ void topk_keys(const uint32_t (&key)[E], Idx idx, int k, int32_t* __restrict__ out, int cap,
                          TopkRegShared& sh) {
  static_assert(NT == 256, "topk_keys: 256 threads");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lo = tid * E;
  for (int i = tid; i < 4 * 256; i += NT) sh.hist[i >> 8][i & 255] = 0;
  __syncthreads();
  // first digit: every key takes part, and the keys of a row mostly share
  // their top byte, so the lanes of the most common bins are counted
  // together
  #pragma unroll
  for (int e = 0; e < E; ++e) hist_add(sh.hist[wave], true, key[e] >> 24);
  __syncthreads();
  pick_digit(sh.hist[0][tid] + sh.hist[1][tid] + sh.hist[2][tid] + sh.hist[3][tid], k, 0u, 0u, 24, sh.scan,
             &sh.prefix, &sh.mask, &sh.remaining);
  for (int shift = 16; shift >= 0; shift -= 8) {
    for (int i = tid; i < 4 * 256; i += NT) sh.hist[i >> 8][i & 255] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix, mask = sh.mask;
    const int rem = sh.remaining;
    // later digits: few keys still match, so a wave with none skips
    #pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool mt = (key[e] & mask) == prefix;
      if (__ballot(mt) != 0ull && mt) atomicAdd(&sh.hist[wave][(key[e] >> shift) & 255u], 1);
    }
    __syncthreads();
    const int tot = sh.hist[0][tid] + sh.hist[1][tid] + sh.hist[2][tid] + sh.hist[3][tid];
    pick_digit(tot, rem, prefix, mask, shift, sh.scan, &sh.prefix, &sh.mask, &sh.remaining);
  }
  const uint32_t T = sh.prefix;
  const int need_eq = sh.remaining;     // elements equal to T that are taken
  int n_gt = 0, n_eq = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) { n_gt += key[e] > T; n_eq += key[e] == T; }
  int tot_eq;
  const int eq_rank0 = block_scan_excl<NT>(n_eq, sh.scan, &tot_eq);
  const int take_eq = max(0, min(n_eq, need_eq - eq_rank0));
  int tot_out;
  int pos = block_scan_excl<NT>(n_gt + take_eq, sh.scan, &tot_out);
  int eq_seen = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    bool sel = key[e] > T;
    if (!sel && key[e] == T) { sel = eq_seen < take_eq; ++eq_seen; }
    if (sel) out[pos++] = idx(lo + e);
  }
  for (int i = k + tid; i < cap; i += NT) out[i] = -1;
  __syncthreads();
}

// Outputs of the cases without a selection: k <= 0 (none taken) or k >= n
// (all taken).  Returns false when a selection is needed.
template <int NT, typename Idx>
__device__ bool topk_trivial(Idx idx, int n, int k, int32_t* __restrict__ out, int cap) {
  const int tid = threadIdx.x;
  if (k <= 0) {
    for (int i = tid; i < cap; i += NT) out[i] = -1;
    __syncthreads();
    return true;
  }
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out[i] = idx(i);
    for (int i = n + tid; i < cap; i += NT) out[i] = -1;
    __syncthreads();
    return true;
  }
  return false;
}

// Loads the keys of get(lo .. lo + E - 1) (key 0 past n).
template <int E, typename Get>
__device__ __forceinline__ void load_keys(Get get, int n, uint32_t (&key)[E]) {
  const int lo = (int)threadIdx.x * E;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t x = order_key(get(lo + e));
    key[e] = lo + e < n ? x : 0u;
  }
}

template <int NT, int E, typename Get, typename Idx>
__device__ void block_topk_reg(Get get, Idx idx, int n, int k, int32_t* __restrict__ out, int cap,
                               TopkRegShared& sh) {
  k = min(k, n);
  if (topk_trivial<NT>(idx, n, k, out, cap)) return;
  uint32_t key[E];
  load_keys<E>(get, n, key);
  topk_keys<NT, E>(key, idx, k, out, cap, sh);
}
template <int NT, int E, typename Get>
__device__ void block_topk_reg(Get get, int n, int k, int32_t* __restrict__ out, int cap, TopkRegShared& sh) {
  block_topk_reg<NT, E>(get, [](int i) { return i; }, n, k, out, cap, sh);
}

// The float whose order_key is key (order_key is a bijection on bit patterns).
__device__ __forceinline__ float key_float(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// The r-th largest (1 <= r <= 256) of the 256 keys x, one per thread, by the
// same four radix passes.
__device__ __forceinline__ uint32_t block_kth_key(uint32_t x, int r, TopkRegShared& sh) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) sh.hist[i >> 8][i & 255] = 0;
  __syncthreads();
  hist_add(sh.hist[wave], true, x >> 24);
  __syncthreads();
  pick_digit(sh.hist[0][tid] + sh.hist[1][tid] + sh.hist[2][tid] + sh.hist[3][tid], r, 0u, 0u, 24, sh.scan,
             &sh.prefix, &sh.mask, &sh.remaining);
  for (int shift = 16; shift >= 0; shift -= 8) {
    for (int i = tid; i < 4 * 256; i += 256) sh.hist[i >> 8][i & 255] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix, mask = sh.mask;
    const int rem = sh.remaining;
    const bool mt = (x & mask) == prefix;
    if (__ballot(mt) != 0ull && mt) atomicAdd(&sh.hist[wave][(x >> shift) & 255u], 1);
    __syncthreads();
    const int tot = sh.hist[0][tid] + sh.hist[1][tid] + sh.hist[2][tid] + sh.hist[3][tid];
    pick_digit(tot, rem, prefix, mask, shift, sh.scan, &sh.prefix, &sh.mask, &sh.remaining);
  }
  return sh.prefix;
}

}  // namespace minf
