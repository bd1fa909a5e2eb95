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
#include "kernels.h"
#include "topk.h"

namespace minf {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

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
  float* dst;
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
    dst = P.kbar + ((size_t)z * P.nq + u) * DH;
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
    dst[threadIdx.x] = sum / (float)(r1 - r0);
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

// grid (items per tile, tiles, batch): causal scores R = scale * Qbar Kbar^T on
// the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  A work-group holds the 128
// query blocks of one tile, wave w the 32 blocks U = 4 tile + w, whose pooled
// rows stay in registers for the whole item (the contraction is only dh
// long, so operands, not products, are the cost to hide); it sweeps pairs of
// 32-block column groups (V0, V0 + 1) from the item's first pair to its last,
// each pair's 64 pooled key rows copied once into LDS for the four waves,
// double-buffered: the next pair's copies are issued before the current
// products.  A tile's pairs are split into items of at most `S` pairs,
// heaviest tiles first, so the grid stays balanced.  Lane (m, hh) of a product
// holds element k of row m, and the contraction index is permuted alike for
// both operands, k = k0 + 4 hh + s at step s of the 8-wide slab k0, so one
// 16-byte read per row and lane feeds four steps; each score is one chain of
// products in ascending slab order.  LDS rows are stored in 16-byte pieces
// at position piece ^ (row & 7), so the eight lanes of one LDS read phase hit
// different banks.
//
// One counter tracks both loads and stores, in issue order.  Every step
// issues exactly 32 score stores per wave after its copies (buffer stores:
// a score outside the causal triangle or past nq gets an offset beyond the
// buffer's end and is dropped, so no store depends on a branch), and the
// wait before the step's barrier leaves those 32 in flight: the copies have
// landed, the stores keep draining under the next step's products.
template <int DH>
__global__ __launch_bounds__(256) void bs_score_kernel(BsParams P, BsBatch batch, int S, int ntiles) {
  constexpr int CH = DH / 4;       // 16-byte pieces per row
  constexpr int NG = DH / 8;       // 8-wide slabs
  constexpr int NI = 64 * CH / 256;   // copies per lane and pair
  const int T = ntiles - 1 - (int)blockIdx.y;
  const int npairs = 2 * T + 2;
  const int j0 = (int)blockIdx.x * S;
  if (j0 >= npairs) return;
  const int j1 = min(j0 + S, npairs);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the buffer resource below is scalar
  const int m = lane & 31, hh = lane >> 5;
  const int U = 4 * T + wave;
  const int bh = batch.bh[blockIdx.z];
  const int b = bh / P.Hq, h = bh % P.Hq;
  const int kv = h / (P.Hq / P.Hkv);
  const int nq = P.nq;
  const float* A = P.qbar + (size_t)bh * nq * DH;
  const float* Bm = P.kbar + ((size_t)b * P.Hkv + kv) * nq * DH;
  __shared__ floatx4 sb[2][64 * CH];
  const uint32_t sbase = (uint32_t)(uintptr_t)&sb[0][0];

  // the copies of pair j into buffer buf: copy i of wave w fills pieces
  // 256 i + 64 w + lane, i.e. row r = piece / CH at position piece % CH,
  // which holds the row's piece (position ^ (r & 7))
  auto copy_pair = [&](int j, int buf) {
    #pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = 256 * i + 64 * wave + lane;
      const int r = pos / CH;
      const int c = (pos % CH) ^ (r & 7);
      const int row = min(64 * j + r, nq - 1);     // rows past nq: computed, never stored
      const uint32_t dst = __builtin_amdgcn_readfirstlane(sbase + (uint32_t)(buf * 64 * CH + 256 * i + 64 * wave) * 16);
      copy_piece(Bm, (uint32_t)((row * DH + 4 * c) * 4), dst);
    }
  };
  copy_pair(j0, 0);
  floatx4 a[NG];
  {
    const float* pa = A + (size_t)min(32 * U + m, nq - 1) * DH + 4 * hh;
    #pragma unroll
    for (int g = 0; g < NG; ++g) a[g] = *reinterpret_cast<const floatx4*>(pa + 8 * g);
  }
  // everything above has landed (a real wait instruction, so that the
  // compiler knows the query rows need no wait inside the sweep)
  __builtin_amdgcn_s_waitcnt(0x0f70);    // vmcnt(0)
  __syncthreads();

  // this wave's 32 rows of R; a score's byte offset within them, or an
  // offset past their end when it is not stored
  const uint32_t rows_bytes = (uint32_t)(32 * nq * 4);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      P.scores + ((size_t)blockIdx.z * nq + (size_t)32 * U) * nq, 0, (int)rows_bytes, 0x00020000);
  const float scale = P.scale;
  auto store_block = [&](const floatx16& acc, int V) {
    // lane (m, hh), register r of a 32x32 product: row 8 (r / 4) + 4 hh + r % 4, column m
    const int vv = 32 * V + m;
    #pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ul = 8 * (r >> 2) + 4 * hh + (r & 3);
      const int uu = 32 * U + ul;
      const uint32_t off = (uu < nq && vv <= uu) ? (uint32_t)((ul * nq + vv) * 4) : 0x7ffffff0u;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, scale * acc[r]), rsrc, (int)off, 0, 0);
    }
  };
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    const int V0 = 2 * j;
    // the other buffer was read in the previous step, before its barrier
    if (j + 1 < j1) copy_pair(j + 1, buf ^ 1);
    const floatx4* s0 = &sb[buf][m * CH];
    const floatx4* s1 = &sb[buf][(32 + m) * CH];
    floatx16 acc0, acc1;
    #pragma unroll
    for (int r = 0; r < 16; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; }
    if (V0 + 1 <= U) {
      #pragma unroll
      for (int g = 0; g < NG; ++g) {
        const floatx4 b0 = s0[(2 * g + hh) ^ (m & 7)];
        const floatx4 b1 = s1[(2 * g + hh) ^ (m & 7)];
        #pragma unroll
        for (int st = 0; st < 4; ++st) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g][st], b0[st], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g][st], b1[st], acc1, 0, 0, 0);
        }
      }
    } else if (V0 <= U) {
      #pragma unroll
      for (int g = 0; g < NG; ++g) {
        const floatx4 b0 = s0[(2 * g + hh) ^ (m & 7)];
        #pragma unroll
        for (int st = 0; st < 4; ++st) acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g][st], b0[st], acc0, 0, 0, 0);
      }
    }
    // blocks past U (the diagonal pair) store nothing: every offset is out of range
    store_block(acc0, V0);
    store_block(acc1, V0 + 1);
    asm volatile("s_waitcnt vmcnt(32)\n\ts_barrier" ::: "memory");
  }
}

// grid (nq, batch): exact top-k of row u over v <= u, the row held in
// registers (E = ceil(nq / 256) scores per thread at most; a row of n = u + 1
// scores takes the smallest of E/4, E/2 and E that covers it).  The selection
// gives each thread consecutive scores; read that way straight from memory,
// one load instruction of a wave would touch 64 cache lines, so the row is
// first copied into LDS with consecutive lanes on consecutive scores (one
// padding word per 32 keeps the per-thread reads free of bank conflicts).
template <int E>
__global__ __launch_bounds__(256) void bs_topk_kernel(BsParams P, BsBatch batch) {
  const int u = blockIdx.x;
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
  if (E >= 16 && n <= 64 * E) block_topk_reg<256, (E >= 16 ? E / 4 : E)>(get, n, k, out, (int)P.max_kb, sh);
  else if (E >= 8 && n <= 128 * E) block_topk_reg<256, (E >= 8 ? E / 2 : E)>(get, n, k, out, (int)P.max_kb, sh);
  else block_topk_reg<256, E>(get, n, k, out, (int)P.max_kb, sh);
  if (threadIdx.x == 0) P.blk_cnt[(size_t)bh * P.nq + u] = k;
}

template <int E>
static void launch_topk(const BsParams& p, const BsBatch& batch, hipStream_t st) {
  hipLaunchKernelGGL(bs_topk_kernel<E>, dim3(p.nq, batch.count), dim3(256), 0, st, p, batch);
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
    // pairs per score item: the longest that still gives about three items
    // per resident work-group slot (two per CU)
    int S = 4;
    for (int cand : {16, 8}) {
      int64_t items = 0;
      for (int t = 0; t < tiles; ++t) items += (2 * t + 2 + cand - 1) / cand;
      if (items * batch.count >= 3 * 512) { S = cand; break; }
    }
    const int per_tile = (2 * tiles + S - 1) / S;
    hipLaunchKernelGGL((bs_score_kernel<DH>), dim3(per_tile, tiles, batch.count), dim3(256), 0, st, p, batch, S, tiles);
    const int64_t per = (p.nq + 255) / 256;   // scores per thread
    if (per <= 4) launch_topk<4>(p, batch, st);
    else if (per <= 8) launch_topk<8>(p, batch, st);
    else if (per <= 16) launch_topk<16>(p, batch, st);
    else if (per <= 32) launch_topk<32>(p, batch, st);
    else if (per <= 64) launch_topk<64>(p, batch, st);
    else launch_topk<128>(p, batch, st);
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
