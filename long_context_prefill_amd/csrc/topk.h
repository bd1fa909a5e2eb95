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

struct TopkShared {
  int hist[256];
  int scan[17];
  uint32_t prefix, mask;
  int remaining;
};

// Selects the top min(k, n) of get(0..n-1) and writes their indices,
// ascending, to out[0..); out[min(k,n) .. cap) is filled with -1.
template <int NT, int E, typename Get>
__device__ void block_topk(Get get, int n, int k, int32_t* __restrict__ out, int cap, TopkShared& sh) {
  const int tid = threadIdx.x;
  k = min(k, n);
  if (k <= 0) {
    for (int i = tid; i < cap; i += NT) out[i] = -1;
    return;
  }
  if (tid == 0) { sh.prefix = 0; sh.mask = 0; sh.remaining = k; }
  if (k < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = sh.prefix, mask = sh.mask;
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = order_key(get(i));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, rem = sh.remaining, dg = 0;
        for (dg = 255; dg > 0; --dg) {
          const int c = sh.hist[dg];
          if (cum + c >= rem) break;
          cum += c;
        }
        sh.remaining = rem - cum;
        sh.prefix = prefix | ((uint32_t)dg << shift);
        sh.mask = mask | (0xffu << shift);
      }
      __syncthreads();
    }
  } else {
    if (tid == 0) { sh.prefix = 0; sh.mask = 0xffffffffu; sh.remaining = n; }   // take all
  }
  __syncthreads();
  const uint32_t T = sh.prefix;
  const bool take_all = (k >= n);
  const int need_eq = sh.remaining;   // elements equal to T that are taken
  int carry_eq = 0, carry_out = 0;
  for (int base = 0; base < n; base += NT * E) {
    const int lo = base + tid * E;
    int n_eq = 0, n_gt = 0;
    #pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lo + e;
      if (i < n) {
        const uint32_t key = order_key(get(i));
        if (take_all || key > T) ++n_gt;
        else if (key == T) ++n_eq;
      }
    }
    int tot_eq;
    const int eq_rank0 = carry_eq + block_scan_excl<NT>(n_eq, sh.scan, &tot_eq);
    const int take_eq = max(0, min(n_eq, need_eq - eq_rank0));
    int tot_out;
    int pos = carry_out + block_scan_excl<NT>(n_gt + take_eq, sh.scan, &tot_out);
    int eq_seen = 0;
    #pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lo + e;
      if (i < n) {
        const uint32_t key = order_key(get(i));
        bool sel = take_all || key > T;
        if (!sel && key == T) { sel = eq_seen < take_eq; ++eq_seen; }
        if (sel) out[pos++] = i;
      }
    }
    carry_eq += tot_eq;
    carry_out += tot_out;
  }
  for (int i = k + tid; i < cap; i += NT) out[i] = -1;
  __syncthreads();
}

}  // namespace minf
