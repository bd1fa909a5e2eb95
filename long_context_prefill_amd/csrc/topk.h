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
  int hist[16][256];   // one histogram per wave (fewer colliding LDS atomics)
  int scan[17];
  uint32_t prefix, mask;
  int remaining;
};

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
    constexpr int NW = NT / 64;
    static_assert(NW <= 16 && NT >= 256, "block_topk: 256..1024 threads");
    const int wave = tid >> 6;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < NW * 256; i += NT) sh.hist[i >> 8][i & 255] = 0;
      __syncthreads();
      const uint32_t prefix = sh.prefix, mask = sh.mask;
      const int rem = sh.remaining;
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = order_key(get(i));
        if ((key & mask) == prefix) atomicAdd(&sh.hist[wave][(key >> shift) & 255u], 1);
      }
      __syncthreads();
      int tot = 0;
      if (tid < 256)
        for (int w = 0; w < NW; ++w) tot += sh.hist[w][tid];
      pick_digit(tot, rem, prefix, mask, shift, sh.scan, &sh.prefix, &sh.mask, &sh.remaining);
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

// The same selection over a plain fp32 array, read with 16-byte loads (when
// it is 16-byte aligned), four in flight per thread: thread t handles the
// groups of 4 elements t, t + NT, ...; the ordered compaction walks the array
// in tiles of NT * 16 elements, thread t owning 16 consecutive ones.
template <int NT>
__device__ void block_topk_array(const float* __restrict__ src, int n, int k, int32_t* __restrict__ out, int cap,
                                 TopkShared& sh) {
  const int tid = threadIdx.x;
  k = min(k, n);
  if (k <= 0) {
    for (int i = tid; i < cap; i += NT) out[i] = -1;
    __syncthreads();
    return;
  }
  const floatx4* src4 = reinterpret_cast<const floatx4*>(src);
  // whole groups of 4 read as vectors when src is 16-byte aligned; an
  // unaligned array (ragged n, or a caller's buffer) is read element by element
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const int n4 = aligned ? (n >> 2) : 0;
  auto key_at = [&](int i) { return order_key(src[i]); };
  if (tid == 0) { sh.prefix = 0; sh.mask = 0; sh.remaining = k; }
  if (k < n) {
    constexpr int NW = NT / 64;
    const int wave = tid >> 6;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < NW * 256; i += NT) sh.hist[i >> 8][i & 255] = 0;
      __syncthreads();
      const uint32_t prefix = sh.prefix, mask = sh.mask;
      const int rem = sh.remaining;
      auto count = [&](uint32_t key) {
        if ((key & mask) == prefix) atomicAdd(&sh.hist[wave][(key >> shift) & 255u], 1);
      };
      int g = tid;
      for (; g + 3 * NT < n4; g += 4 * NT) {
        floatx4 x[4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) x[a] = src4[g + a * NT];
        #pragma unroll
        for (int a = 0; a < 4; ++a)
          #pragma unroll
          for (int e = 0; e < 4; ++e) count(order_key(x[a][e]));
      }
      for (; g < n4; g += NT) {
        const floatx4 x = src4[g];
        #pragma unroll
        for (int e = 0; e < 4; ++e) count(order_key(x[e]));
      }
      for (int i = 4 * n4 + tid; i < n; i += NT) count(key_at(i));
      __syncthreads();
      int tot = 0;
      if (tid < 256)
        for (int w = 0; w < NW; ++w) tot += sh.hist[w][tid];
      pick_digit(tot, rem, prefix, mask, shift, sh.scan, &sh.prefix, &sh.mask, &sh.remaining);
    }
  } else {
    if (tid == 0) { sh.prefix = 0; sh.mask = 0xffffffffu; sh.remaining = n; }   // take all
  }
  __syncthreads();
  const uint32_t T = sh.prefix;
  const bool take_all = (k >= n);
  const int need_eq = sh.remaining;
  int carry_eq = 0, carry_out = 0;
  constexpr int E = 16;
  for (int base = 0; base < n; base += NT * E) {
    const int lo = base + tid * E;
    uint32_t key[E];
    #pragma unroll
    for (int a = 0; a < E / 4; ++a) {
      if (aligned && lo + 4 * a + 3 < n) {
        const floatx4 x = src4[(lo >> 2) + a];
        #pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * a + e] = order_key(x[e]);
      } else {
        #pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * a + e] = lo + 4 * a + e < n ? key_at(lo + 4 * a + e) : 0u;
      }
    }
    int n_eq = 0, n_gt = 0;
    #pragma unroll
    for (int e = 0; e < E; ++e)
      if (lo + e < n) {
        if (take_all || key[e] > T) ++n_gt;
        else if (key[e] == T) ++n_eq;
      }
    int tot_eq;
    const int eq_rank0 = carry_eq + block_scan_excl<NT>(n_eq, sh.scan, &tot_eq);
    const int take_eq = max(0, min(n_eq, need_eq - eq_rank0));
    int tot_out;
    int pos = carry_out + block_scan_excl<NT>(n_gt + take_eq, sh.scan, &tot_out);
    int eq_seen = 0;
    #pragma unroll
    for (int e = 0; e < E; ++e) {
      if (lo + e < n) {
        bool sel = take_all || key[e] > T;
        if (!sel && key[e] == T) { sel = eq_seen < take_eq; ++eq_seen; }
        if (sel) out[pos++] = lo + e;
      }
    }
    carry_eq += tot_eq;
    carry_out += tot_out;
  }
  for (int i = k + tid; i < cap; i += NT) out[i] = -1;
  __syncthreads();
}

// The same selection for up to NT * E elements held in registers: thread t
// reads elements [t*E, t*E + E) once; the four radix passes and the ordered
// compaction work on those registers.  `get(i)` is called once per element.
struct TopkRegShared {
  int hist[4][256];
  int scan[17];
  uint32_t prefix, mask;
  int remaining;
};

template <int NT, int E, typename Get>
__device__ void block_topk_reg(Get get, int n, int k, int32_t* __restrict__ out, int cap, TopkRegShared& sh) {
  static_assert(NT == 256, "block_topk_reg: 256 threads");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  k = min(k, n);
  const int lo = tid * E;
  if (k <= 0) {
    for (int i = tid; i < cap; i += NT) out[i] = -1;
    __syncthreads();
    return;
  }
  if (k >= n) {
    // every element is taken
    for (int i = tid; i < n; i += NT) out[i] = i;
    for (int i = n + tid; i < cap; i += NT) out[i] = -1;
    __syncthreads();
    return;
  }
  uint32_t key[E];
  #pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (lo + e < n) ? order_key(get(lo + e)) : 0u;
  if (tid == 0) { sh.prefix = 0; sh.mask = 0; sh.remaining = k; }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 4 * 256; i += NT) sh.hist[i >> 8][i & 255] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix, mask = sh.mask;
    const int rem = sh.remaining;
    #pragma unroll
    for (int e = 0; e < E; ++e)
      if (lo + e < n && (key[e] & mask) == prefix) atomicAdd(&sh.hist[wave][(key[e] >> shift) & 255u], 1);
    __syncthreads();
    const int tot = sh.hist[0][tid] + sh.hist[1][tid] + sh.hist[2][tid] + sh.hist[3][tid];
    pick_digit(tot, rem, prefix, mask, shift, sh.scan, &sh.prefix, &sh.mask, &sh.remaining);
  }
  const uint32_t T = sh.prefix;
  const int need_eq = sh.remaining;     // elements equal to T that are taken
  int n_gt = 0, n_eq = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e)
    if (lo + e < n) { n_gt += key[e] > T; n_eq += key[e] == T; }
  int tot_eq;
  const int eq_rank0 = block_scan_excl<NT>(n_eq, sh.scan, &tot_eq);
  const int take_eq = max(0, min(n_eq, need_eq - eq_rank0));
  int tot_out;
  int pos = block_scan_excl<NT>(n_gt + take_eq, sh.scan, &tot_out);
  int eq_seen = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lo + e < n) {
      bool sel = key[e] > T;
      if (!sel && key[e] == T) { sel = eq_seen < take_eq; ++eq_seen; }
      if (sel) out[pos++] = lo + e;
    }
  }
  for (int i = k + tid; i < cap; i += NT) out[i] = -1;
  __syncthreads();
}

}  // namespace minf
