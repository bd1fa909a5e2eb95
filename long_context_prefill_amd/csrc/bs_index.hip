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
// from HBM; a tiled fp32 product on the matrix cores writes the causal score
// tiles of a batch of heads into the workspace (so the score matrix never has to be resident for
// the whole layer); one work-group per (head, query block) then runs the
// exact radix top-k on its row.
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

// grid (tiles_v, tiles_u, batch): 128x128 causal tiles of R = scale * Qbar Kbar^T
// on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  Wave w computes the
// 64x64 quarter (w / 2, w % 2) as 2x2 products of 32x32; the waves share
// nothing, so a quarter wholly above the diagonal simply exits.  Operands come
// straight from the pooled rows (they stay in L2): lane (m, hh) of a product
// holds element k of row m, and the contraction index is permuted alike for
// both operands, k = k0 + 4 hh + s at step s of the 8-wide slab k0, so one
// 16-byte load per row and lane feeds four steps.
template <int DH>
__global__ __launch_bounds__(256) void bs_score_kernel(BsParams P, BsBatch batch) {
  const int tv = blockIdx.x, tu = blockIdx.y;
  if (tv > tu) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 31, hh = lane >> 5;
  const int u0 = 128 * tu + 64 * (wave >> 1), v0 = 128 * tv + 64 * (wave & 1);
  if (v0 > u0 + 63 || u0 >= P.nq) return;
  const int bh = batch.bh[blockIdx.z];
  const int b = bh / P.Hq, h = bh % P.Hq;
  const int kv = h / (P.Hq / P.Hkv);
  const float* A = P.qbar + (size_t)bh * P.nq * DH;
  const float* Bm = P.kbar + ((size_t)b * P.Hkv + kv) * P.nq * DH;
  float* R = P.scores + (size_t)blockIdx.z * P.nq * P.nq;
  // rows past nq are clamped to the last row: computed, never stored
  const float* pa[2];
  const float* pb[2];
  #pragma unroll
  for (int i = 0; i < 2; ++i) {
    pa[i] = A + (size_t)min(u0 + 32 * i + m, P.nq - 1) * DH + 4 * hh;
    pb[i] = Bm + (size_t)min(v0 + 32 * i + m, P.nq - 1) * DH + 4 * hh;
  }
  floatx16 acc[2][2];
  #pragma unroll
  for (int i = 0; i < 2; ++i)
    #pragma unroll
    for (int jx = 0; jx < 2; ++jx)
      #pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][jx][r] = 0.f;
  #pragma unroll 4
  for (int k0 = 0; k0 < DH; k0 += 8) {
    floatx4 xa[2], xb[2];
    #pragma unroll
    for (int i = 0; i < 2; ++i) {
      xa[i] = *reinterpret_cast<const floatx4*>(pa[i] + k0);
      xb[i] = *reinterpret_cast<const floatx4*>(pb[i] + k0);
    }
    #pragma unroll
    for (int st = 0; st < 4; ++st)
      #pragma unroll
      for (int i = 0; i < 2; ++i)
        #pragma unroll
        for (int jx = 0; jx < 2; ++jx)
          acc[i][jx] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[i][st], xb[jx][st], acc[i][jx], 0, 0, 0);
  }
  // lane (m, hh), register r of a 32x32 product: row 8 (r / 4) + 4 hh + r % 4, column m
  #pragma unroll
  for (int i = 0; i < 2; ++i)
    #pragma unroll
    for (int jx = 0; jx < 2; ++jx) {
      const int vv = v0 + 32 * jx + m;
      #pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int uu = u0 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (uu < P.nq && vv <= uu) R[(size_t)uu * P.nq + vv] = P.scale * acc[i][jx][r];
      }
    }
}

// grid (nq, batch): exact top-k of row u over v <= u, the row held in
// registers (E = ceil(nq / 256) scores per thread).
template <int E>
__global__ __launch_bounds__(256) void bs_topk_kernel(BsParams P, BsBatch batch) {
  const int u = blockIdx.x;
  const int bh = batch.bh[blockIdx.y];
  const int h = bh % P.Hq;
  __shared__ TopkRegShared sh;
  const float* row = P.scores + ((size_t)blockIdx.y * P.nq + u) * P.nq;
  const int force = P.ht.b[h];
  const float inf = __builtin_huge_valf();
  const int k = min(P.ht.a[h], u + 1);
  int32_t* out = P.blk_idx + ((size_t)bh * P.nq + u) * P.max_kb;
  block_topk_reg<256, E>(
      [&](int v) {
        if (((force & MINF_FORCE_FIRST_BLOCK) && v == 0) || ((force & MINF_FORCE_DIAG_BLOCK) && v == u)) return inf;
        return row[v];
      },
      u + 1, k, out, (int)P.max_kb, sh);
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
    hipLaunchKernelGGL((bs_score_kernel<DH>), dim3(tiles, tiles, batch.count), dim3(256), 0, st, p, batch);
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
