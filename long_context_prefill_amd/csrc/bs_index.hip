// Block-Sparse index estimation.
//
// PaperTrace 2.1.2 "MInference", section 2 (Eq. 6 and the mean-pooling proxy)
// and blog-zz7 "LLM模型之MInference" section 2.3.2: Q and K are mean-pooled
// over 64-token blocks, the block scores r_uv = scale * Qbar_u . Kbar_v are
// formed for v <= u, and every query block keeps its top-k_b key blocks.
// Forced blocks (first / diagonal) take an infinite score, so they occupy
// budget slots.  Everything is fp32 and free of floating-point atomics.
//
// GPU plan: a pooling pass streams Q (BS heads) and K (their KV heads) once
// from HBM; an fp32 product on the matrix cores writes the causal scores of a
// batch of heads into the workspace (so the score matrix never has to be
// resident for the whole layer); one work-group per (head, query block) then
// runs the exact radix top-k on its row.
#include <type_traits>

#include "kernels.h"
#include "topk.h"

namespace minf {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx16 mma32(u32x4 a, u32x4 b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Round to the nearest bf16, ties to even (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }

// x = t0 + t1 + t2 + e with bf16 terms: each term is the nearest bf16 to
// what the earlier ones leave (the differences are exact in fp32), so
// |e| <= 2^-24 |x| up to the spacing of the smallest term.
__device__ __forceinline__ void split3_bf16(float x, uint16_t (&t)[3]) {
  t[0] = bf16_rne(x);
  const float r1 = x - bf16_f32(t[0]);
  t[1] = bf16_rne(r1);
  t[2] = bf16_rne(r1 - bf16_f32(t[1]));
}

struct BsBatch {
  int32_t count;
  int32_t bh[64];      // b * Hq + h of each head in this batch
};

// grid (nq, B*Hq + B*Hkv): mean of each 64-row block of Q (BS heads) and K.
// Thread t reads 16 bytes (columns 16/sizeof(T) * (t % CPR) ..) of rows
// t / CPR, + RG, ...; the row groups are then summed through LDS in a fixed
// order.
template <typename T, int DH>
__global__ __launch_bounds__(256) void bs_pool_kernel(BsParams P, uint64_t kv_used) {
  constexpr int EPL = 16 / (int)sizeof(T);   // elements per 16-byte load
  constexpr int CPR = DH / EPL;              // loads per row
  constexpr int RG = 256 / CPR;              // row groups
  const int u = blockIdx.x;
  const int y = blockIdx.y;
  const int BHq = P.B * P.Hq;
  const T* src;
  float* dst = nullptr;
  uint16_t* dst3 = nullptr;
  if (y < BHq) {
    const int h = y % P.Hq;
    if (P.ht.kind[h] != MINF_BSPARSE) return;
    src = reinterpret_cast<const T*>(P.Q) + (size_t)y * P.n * DH;
    dst = P.qbar + ((size_t)y * P.nq + u) * DH;
  } else {
    const int z = y - BHq;
    const int kv = z % P.Hkv;
    if (!((kv_used >> kv) & 1ull)) return;
    src = reinterpret_cast<const T*>(P.K) + (size_t)z * P.n * DH;
    dst3 = P.kbar3 + ((size_t)z * P.nq + u) * 3 * DH;
  }
  const int r0 = 64 * u, r1 = min(r0 + 64, P.n);
  const int c = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  float acc[EPL];
  #pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int r = r0 + rg; r < r1; r += RG) {
    if constexpr (sizeof(T) == 2) {
      // the four packed dwords are read as separate scalars (bit-casting
      // elements extracted from a loaded vector has been miscompiled)
      const uint32_t* w = reinterpret_cast<const uint32_t*>(src + (size_t)r * DH + c * EPL);
      const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
      acc[0] += __builtin_bit_cast(float, w0 << 16); acc[1] += __builtin_bit_cast(float, w0 & 0xffff0000u);
      acc[2] += __builtin_bit_cast(float, w1 << 16); acc[3] += __builtin_bit_cast(float, w1 & 0xffff0000u);
      acc[4] += __builtin_bit_cast(float, w2 << 16); acc[5] += __builtin_bit_cast(float, w2 & 0xffff0000u);
      acc[6] += __builtin_bit_cast(float, w3 << 16); acc[7] += __builtin_bit_cast(float, w3 & 0xffff0000u);
    } else {
      const floatx4 x = *reinterpret_cast<const floatx4*>(src + (size_t)r * DH + c * EPL);
      #pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += x[e];
    }
  }
  __shared__ float part[RG][DH + 1];
  #pragma unroll
  for (int e = 0; e < EPL; ++e) part[rg][c * EPL + e] = acc[e];
  __syncthreads();
  if ((int)threadIdx.x < DH) {
    float sum = 0.f;
    for (int g = 0; g < RG; ++g) sum += part[g][threadIdx.x];
    const float mean = sum / (float)(r1 - r0);
    if (dst) {
      dst[threadIdx.x] = mean;
    } else {
      uint16_t t3[3];
      split3_bf16(mean, t3);
      #pragma unroll
      for (int p = 0; p < 3; ++p) dst3[p * DH + threadIdx.x] = t3[p];
    }
  }
}

// One direct global->LDS copy of 16 bytes per lane: lane l's piece lands at
// LDS byte address dst + 16 l.  Inline assembly, so the compiler neither
// waits for it nor orders LDS reads after it; completion is waited for
// explicitly (M0 is declared clobbered, one wait state after writing it).
__device__ __forceinline__ void copy_piece(const float* base, uint32_t voff, uint32_t dst) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(dst)
      : "memory", "m0");
}

// grid (items per tile, tiles, batch): causal scores R = scale * Qbar Kbar^T.
// The products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with
// every fp32 operand split into three bf16 terms (hi, mid, lo; the key rows
// come split from the pooling pass): a . b is summed as hi.hi + (hi.mid +
// mid.hi) + (hi.lo + mid.mid + lo.hi), whose dropped terms and splitting
// residue are below 2^-22 of |a| |b| per element, fp32-level error at a
// sixth of the fp32 matrix instruction's time.  A work-group holds the 128
// query blocks of one tile, wave w the 32 blocks U = 4 tile + w, whose three
// terms stay in registers for the whole item; it sweeps the causal key
// blocks V = 0 .. 4 tile + 3 in steps of 32, each step's 32 split key rows
// copied once into LDS for the four waves, double-buffered: the next step's
// copies are issued before the current products.  A tile's steps are split
// into items of at most `S` steps, heaviest tiles first.  Lane (m, hh) of a
// product holds elements 16 s + 8 hh .. + 7 of row m at slab s.  LDS rows
// keep each term's 16-byte pieces at position piece ^ (row & (pieces - 1)),
// so the lanes of one LDS read phase hit different banks.
//
// One counter tracks both loads and stores, in issue order.  Every step
// issues exactly 16 score stores per wave after its copies (buffer stores:
// a score outside the causal triangle or past nq gets an offset beyond the
// buffer's end and is dropped, so no store depends on a branch), and the
// wait before the step's barrier leaves those 16 in flight: the copies have
// landed, the stores keep draining under the next step's products.
template <int DH>
__global__ __launch_bounds__(256) void bs_score_kernel(BsParams P, BsBatch batch, int S, int ntiles) {
  constexpr int NS = DH / 16;         // 16-wide slabs
  constexpr int PC = DH / 8;          // 16-byte pieces per term of a row
  constexpr int RP = 3 * PC;          // pieces per staged row
  constexpr int NI = 32 * RP / 256;   // copies per lane and step
  static_assert(32 * RP % 256 == 0, "whole copies");
  const int T = ntiles - 1 - (int)blockIdx.y;
  const int nsteps = 4 * T + 4;
  const int j0 = (int)blockIdx.x * S;
  if (j0 >= nsteps) return;
  const int j1 = min(j0 + S, nsteps);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the buffer resource below is scalar
  const int m = lane & 31, hh = lane >> 5;
  const int U = 4 * T + wave;
  const int bh = batch.bh[blockIdx.z];
  const int b = bh / P.Hq, h = bh % P.Hq;
  const int kv = h / (P.Hq / P.Hkv);
  const int nq = P.nq;
  const float* A = P.qbar + (size_t)bh * nq * DH;
  const uint16_t* B3 = P.kbar3 + ((size_t)b * P.Hkv + kv) * nq * 3 * DH;
  __shared__ u32x4 sb[2][32 * RP];
  const uint32_t sbase = (uint32_t)(uintptr_t)&sb[0][0];

  // the copies of key block V into buffer buf: copy i of wave w fills pieces
  // 256 i + 64 w + lane, i.e. row r = piece / RP, term q / PC at position
  // q % PC (q = piece % RP), which holds that term's piece
  // (position ^ (r & (PC - 1)))
  auto copy_block = [&](int V, int buf) {
    #pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = 256 * i + 64 * wave + lane;
      const int r = pos / RP, q = pos % RP;
      const int term = q / PC, c = (q % PC) ^ (r & (PC - 1));
      const int row = min(32 * V + r, nq - 1);     // rows past nq: computed, never stored
      const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + (uint32_t)(buf * 32 * RP + 256 * i + 64 * wave) * 16);
      copy_piece(reinterpret_cast<const float*>(B3), (uint32_t)(((row * 3 + term) * DH + 8 * c) * 2), dst);
    }
  };
  copy_block(j0, 0);
  // this wave's pooled query rows as three bf16 terms
  u32x4 a[3][NS];
  {
    const float* pa = A + (size_t)min(32 * U + m, nq - 1) * DH + 8 * hh;
    #pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(pa + 16 * sl);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(pa + 16 * sl + 4);
      uint16_t t[8][3];
      #pragma unroll
      for (int e = 0; e < 4; ++e) { split3_bf16(x0[e], t[e]); split3_bf16(x1[e], t[4 + e]); }
      #pragma unroll
      for (int q = 0; q < 3; ++q)
        #pragma unroll
        for (int e = 0; e < 4; ++e) a[q][sl][e] = (uint32_t)t[2 * e][q] | ((uint32_t)t[2 * e + 1][q] << 16);
    }
  }
  // everything above has landed (a real wait instruction, so that the
  // compiler knows the query terms need no wait inside the sweep)
  __builtin_amdgcn_s_waitcnt(0x0f70);    // vmcnt(0)
  __syncthreads();

  // this wave's 32 rows of R; a score's byte offset within them, or an
  // offset past their end when it is not stored
  const uint32_t rows_bytes = (uint32_t)(32 * nq * 4);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      P.scores + ((size_t)blockIdx.z * nq + (size_t)32 * U) * nq, 0, (int)rows_bytes, 0x00020000);
  const float scale = P.scale;
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    const int V = j;
    // the other buffer was read in the previous step, before its barrier
    if (j + 1 < j1) copy_block(j + 1, buf ^ 1);
    floatx16 c0, c1, c2;
    #pragma unroll
    for (int r = 0; r < 16; ++r) { c0[r] = 0.f; c1[r] = 0.f; c2[r] = 0.f; }
    if (V <= U) {
      const u32x4* srow = &sb[buf][m * RP];
      #pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const int c = (2 * sl + hh) ^ (m & (PC - 1));
        const u32x4 b0 = srow[c], b1 = srow[PC + c], b2 = srow[2 * PC + c];
        c0 = mma32(a[0][sl], b0, c0);
        c1 = mma32(a[0][sl], b1, c1);
        c2 = mma32(a[0][sl], b2, c2);
        c1 = mma32(a[1][sl], b0, c1);
        c2 = mma32(a[1][sl], b1, c2);
        c2 = mma32(a[2][sl], b0, c2);
      }
    }
    // lane (m, hh), register r of a 32x32 product: row 8 (r / 4) + 4 hh + r % 4,
    // column m; a block past U (the diagonal) stores nothing
    const int vv = 32 * V + m;
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ul = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int uu = 32 * U + ul;
      const uint32_t off = (uu < nq && vv <= uu) ? (uint32_t)((ul * nq + vv) * 4) : 0x7ffffff0u;
      const float x = scale * (c0[r] + (c1[r] + c2[r]));
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rsrc, (int)off, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  }
}

// grid (nq, batch): exact top-k of row u over v <= u, the row held in
// registers (E = ceil(nq / 256) scores per thread at most; a row of n = u + 1
// scores takes the smallest of E/4, E/2 and E that covers it).  The selection
// gives each thread consecutive scores; read that way straight from memory,
// one load instruction of a wave would touch 64 cache lines, so the row is
// first copied into LDS with consecutive lanes on consecutive scores (one
// padding word per 32 keeps the per-thread reads free of bank conflicts).
// Top-k of a row staged in LDS (srow, W words), E2 scores per thread.  When
// k is small against n, a sample of the row (each thread's first score)
// bounds the candidates first: Ts is the r-th largest sample, with r about
// three standard deviations above the number of samples expected above the
// k-th largest score.  If at least k scores are >= Ts (then every score >=
// the k-th largest is among them) and they fit, they are copied in index
// order over the staged row and the exact selection runs on them alone (ties
// still go to the lowest index: the copy keeps the order); otherwise it runs
// on the whole row.  Either way the result is the exact top-k.
template <int E2, int W, bool SAMPLE, typename Get>
__device__ void row_topk(Get get, int n, int k, int32_t* __restrict__ out, int cap, TopkRegShared& sh,
                         float* srow) {
  // candidate (key, index) pairs that fit: 1024 or 2048 (E2 >= 8 gives W >=
  // 2112 words)
  constexpr int PAIRS = W / 2 >= 2048 ? 2048 : 1024;
  k = min(k, n);
  auto ident = [](int i) { return i; };
  if (topk_trivial<256>(ident, n, k, out, cap)) return;
  uint32_t key[E2];
  load_keys<E2>(get, n, key);
  // threads past the row contribute key 0, below every real key; r <= ns
  // keeps the threshold a real key, so no slot past n is a candidate
  const int lo = (int)threadIdx.x * E2;
  uint32_t ts = 0;
  int total = 0, pos = 0;
  if (SAMPLE && 4 * k <= n) {
    const int ns = (n + E2 - 1) / E2;
    const float m = (float)k * (float)ns / (float)n;
    const int r = min(ns, (int)(m + 3.0f * __builtin_sqrtf(m)) + 3);
    ts = block_kth_key(key[0], r, sh);
    int nc = 0;
    #pragma unroll
    for (int e = 0; e < E2; ++e) nc += key[e] >= ts;
    pos = block_scan_excl<256>(nc, sh.scan, &total);
  }
  if (total < k || total > PAIRS) {
    topk_keys<256, E2>(key, ident, k, out, cap, sh);
    return;
  }
  // every thread has read its scores (the barriers above): the row's LDS
  // now holds the candidates' keys, then their indices
  uint32_t* ck = reinterpret_cast<uint32_t*>(srow);
  int32_t* ci = reinterpret_cast<int32_t*>(srow) + PAIRS;
  #pragma unroll
  for (int e = 0; e < E2; ++e)
    if (key[e] >= ts) {
      ck[pos] = key[e];
      ci[pos] = lo + e;
      ++pos;
    }
  __syncthreads();
  auto idxc = [&](int i) { return ci[i]; };
  // candidate slots CE t .. CE t + CE - 1 of thread t (below PAIRS); slots
  // past total get key 0
  auto run = [&](auto ce) {
    constexpr int CE = decltype(ce)::value;
    uint32_t kc[CE];
    #pragma unroll
    for (int e = 0; e < CE; ++e) {
      const int i = (int)threadIdx.x * CE + e;
      kc[e] = i < total ? ck[i] : 0u;
    }
    topk_keys<256, CE>(kc, idxc, k, out, cap, sh);
  };
  if (total <= 512) run(std::integral_constant<int, 2>{});
  else if (total <= 1024) run(std::integral_constant<int, 4>{});
  else run(std::integral_constant<int, PAIRS / 256>{});
}

// Rows u0 .. u0 + gridDim.x - 1 of the batch's heads, each at most 256 E
// scores, held E per thread (E_LO for rows of at most 256 E_LO); SAMPLE
// bounds the candidates by a sample first (row_topk).  One launch per
// row-length range, so that every launch stages its rows in an LDS row of
// about their size.
template <int E, int E_LO, bool SAMPLE>
__global__ __launch_bounds__(256) void bs_topk_kernel(BsParams P, BsBatch batch, int u0) {
  const int u = u0 + (int)blockIdx.x;
  const int bh = batch.bh[blockIdx.y];
  const int h = bh % P.Hq;
  __shared__ TopkRegShared sh;
  __shared__ float srow[E * 256 + E * 8];
  const float* row = P.scores + ((size_t)blockIdx.y * P.nq + u) * P.nq;
  const int n = u + 1;
  constexpr int G = E < 16 ? E : 16;     // loads in flight per thread
  #pragma unroll
  for (int e0 = 0; e0 < E; e0 += G) {
    if (256 * e0 >= n) break;
    float x[G];
    #pragma unroll
    for (int e = 0; e < G; ++e) {
      const int v = (int)threadIdx.x + 256 * (e0 + e);
      x[e] = v < n ? row[v] : 0.f;
    }
    #pragma unroll
    for (int e = 0; e < G; ++e) {
      const int v = (int)threadIdx.x + 256 * (e0 + e);
      srow[v + (v >> 5)] = x[e];
    }
  }
  __syncthreads();
  const int force = P.ht.b[h];
  const int k = min(P.ht.a[h], n);
  int32_t* out = P.blk_idx + ((size_t)bh * P.nq + u) * P.max_kb;
  // v < E * 256 stays inside srow; values past n are discarded
  auto get = [&](int v) {
    const float x = srow[v + (v >> 5)];
    const bool forced = ((force & MINF_FORCE_FIRST_BLOCK) && v == 0) || ((force & MINF_FORCE_DIAG_BLOCK) && v == u);
    return forced ? __builtin_huge_valf() : x;
  };
  constexpr int W = E * 256 + E * 8;
  if (E_LO < E && n <= 256 * E_LO) row_topk<E_LO, W, false>(get, n, k, out, (int)P.max_kb, sh, srow);
  else row_topk<E, W, SAMPLE>(get, n, k, out, (int)P.max_kb, sh, srow);
  if (threadIdx.x == 0) P.blk_cnt[(size_t)bh * P.nq + u] = k;
}

// Rows of up to 1024 scores take four per thread, up to 2048 eight (one
// launch); then each doubling of the row length doubles the width, up to 128
// (32768 blocks, the most a Block-Sparse row may hold).  Rows of 2048 to
// 8191 scores bound their candidates by a sample first (the 512K layer's
// Block-Sparse index went from 7.3 to 6.3 ms); on rows of 1024 to 2047 that
// was 10% slower (the radix passes over eight registers cost less than the
// extra passes over the sample), and the widest rows keep the plain path,
// whose registers the sampling would overflow.
static void launch_topk(const BsParams& p, const BsBatch& batch, hipStream_t st) {
  for (int64_t lo = 0; lo < p.nq; lo = lo ? 2 * lo : 2048) {
    const int64_t hi = std::min<int64_t>(lo ? 2 * lo : 2048, p.nq);
    const dim3 grid((unsigned)(hi - lo), batch.count);
    const int u0 = (int)lo;
    if (hi <= 2048) hipLaunchKernelGGL((bs_topk_kernel<8, 4, false>), grid, dim3(256), 0, st, p, batch, u0);
    else if (hi <= 4096) hipLaunchKernelGGL((bs_topk_kernel<16, 16, true>), grid, dim3(256), 0, st, p, batch, u0);
    else if (hi <= 8192) hipLaunchKernelGGL((bs_topk_kernel<32, 32, true>), grid, dim3(256), 0, st, p, batch, u0);
    else if (hi <= 16384) hipLaunchKernelGGL((bs_topk_kernel<64, 64, false>), grid, dim3(256), 0, st, p, batch, u0);
    else hipLaunchKernelGGL((bs_topk_kernel<128, 128, false>), grid, dim3(256), 0, st, p, batch, u0);
  }
}

template <typename T, int DH>
hipError_t launch_t(const BsParams& p, hipStream_t st) {
  uint64_t kv_used = 0;
  for (int h = 0; h < p.Hq; ++h)
    if (p.ht.kind[h] == MINF_BSPARSE) kv_used |= 1ull << (h / (p.Hq / p.Hkv));
  hipLaunchKernelGGL((bs_pool_kernel<T, DH>), dim3(p.nq, p.B * (p.Hq + p.Hkv)), dim3(256), 0, st, p, kv_used);
  BsBatch batch{};
  const int tiles = (p.nq + 127) / 128;
  auto flush = [&]() {
    if (!batch.count) return;
    // key blocks per score item: the longest that still gives about three
    // items per resident work-group slot (two per CU)
    int S = 8;
    for (int cand : {32, 16}) {
      int64_t items = 0;
      for (int t = 0; t < tiles; ++t) items += (4 * t + 4 + cand - 1) / cand;
      if (items * batch.count >= 3 * 512) { S = cand; break; }
    }
    const int per_tile = (4 * tiles + S - 1) / S;
    hipLaunchKernelGGL((bs_score_kernel<DH>), dim3(per_tile, tiles, batch.count), dim3(256), 0, st, p, batch, S, tiles);
    launch_topk(p, batch, st);
    batch.count = 0;
  };
  const int cap = (int)std::min<int64_t>(p.score_heads, 64);
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      if (p.ht.kind[h] != MINF_BSPARSE) continue;
      batch.bh[batch.count++] = b * p.Hq + h;
      if (batch.count == cap) flush();
    }
  flush();
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bs_index(const BsParams& p, hipStream_t st) {
  if (p.in_bf16) return p.dh == 128 ? launch_t<uint16_t, 128>(p, st) : launch_t<uint16_t, 64>(p, st);
  return p.dh == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace minf
