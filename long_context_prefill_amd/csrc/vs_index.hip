// Vertical-Slash index estimation.
//
// PaperTrace 2.1.2 "MInference", section 6.2 (estimating columns and offsets
// from sampled queries) and blog-zz7 "LLM模型之MInference" section 2.3.2 (the
// last queries against all keys): for each VS head h and its last
// L = min(last_q, n) rows i, the proxy weights are the causal softmax
//   a_ij = exp(s_ij - LSE_i),  s_ij = scale * q_i . k_j,  j <= i,
// the column score is c_j = sum_i a_ij and the slash score r_d = sum_i a_{i,i-d};
// the top-v columns and the top-s offsets are kept.
//
// GPU plan:
//  pass 1  every wave takes 256 consecutive keys, forms S^T = K . Q^T for the
//          64 sampled rows with the bf16 (or fp32) matrix cores and keeps a
//          running (max, sum) per row -> per-wave partials;
//  lse     the partials of each row are combined in a fixed order;
//  pass 2  the same S^T tiles are recomputed and turned into exact
//          probabilities; column sums are finished inside the wave (every key
//          belongs to exactly one wave) and diagonal sums are accumulated in
//          registers (lane shifts within 16-lane rows), combined per wave
//          through LDS and written as partials;
//  diag    each offset's two neighbouring partials are added in a fixed order;
//  top-k   exact radix select per (head, score array): one launch per 8-bit
//          digit, each picking the previous digit from its histogram first,
//          then a count and an ordered compaction.
// minf_vs_index_fused runs pass 1, the fold and pass 2 in one launch instead
// (described with its kernel below); the selection is shared.
// No floating-point atomics are used, so two runs give identical bits.
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "topk.h"

namespace minf {

constexpr int kTkSlots = 5;   // select states per top-k array: the start and one after each digit

VsWs vs_workspace(int B, int Hq, int n, int nq) {
  (void)nq;
  VsWs w{};
  const int64_t BH = (int64_t)B * Hq;
  w.nslots = ((int64_t)n + kVsGroupKeys - 1) / kVsGroupKeys * 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  w.part_m = take(BH * 64 * w.nslots * 4);
  w.part_l = take(BH * 64 * w.nslots * 4);
  w.lse2 = take(BH * 64 * 4);
  w.cbuf = take(BH * (size_t)n * 4);
  w.rbuf = take(BH * (size_t)n * 4);
  w.dpart = take(BH * w.nslots * kVsDiagSlots * 4);
  w.sync = take((1 + 2 * BH) * 4);
  w.tk_segs = ((int64_t)n + kTopkSeg - 1) / kTopkSeg;
  w.tk_state = take(2 * BH * kTkSlots * 4 * 4);
  w.tk_hist = take(2 * BH * 4 * 256 * 4);
  w.tk_cnt = take(2 * BH * w.tk_segs * 2 * 4);
  w.total = off;
  return w;
}

namespace {

template <typename T, int DH>
struct ProxyOps {
  static constexpr int KS = (sizeof(T) == 2) ? DH / 32 : DH / 4;
  using QOp = typename std::conditional<(sizeof(T) == 2), u32x4, float>::type;

  // A operand (keys) for 16 keys starting at `key0 + 16*hh`: lane row r16.
  __device__ static __forceinline__ void load_k(const T* Kb, int key, int g, QOp (&k)[KS]) {
    if constexpr (sizeof(T) == 2) {
      const u32x4* p = reinterpret_cast<const u32x4*>(Kb + (size_t)key * DH + g * (DH / 4));
      #pragma unroll
      for (int s = 0; s < KS; ++s) k[s] = p[s];
    } else {
      const floatx4* p = reinterpret_cast<const floatx4*>(Kb + (size_t)key * DH + g * (DH / 4));
      #pragma unroll
      for (int s = 0; s < KS / 4; ++s) {
        floatx4 x = p[s];
        k[4 * s] = x[0]; k[4 * s + 1] = x[1]; k[4 * s + 2] = x[2]; k[4 * s + 3] = x[3];
      }
    }
  }
  __device__ static __forceinline__ void zero(QOp (&q)[KS]) {
    #pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (sizeof(T) == 2) q[s] = u32x4{0, 0, 0, 0};
      else q[s] = 0.f;
    }
  }
  __device__ static __forceinline__ floatx4 dot(const QOp (&k)[KS], const QOp (&q)[KS]) {
    floatx4 a = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (sizeof(T) == 2) a = mma_bf16(k[s], q[s], a);
      else a = mma_f32(k[s], q[s], a);
    }
    return a;
  }
};

// Adds src of lane (l + N) (DPP row_shl:N) or lane (l - N) (row_shr:N) within
// each row of 16 lanes; lanes whose source lies outside the row add 0.
template <int CTRL>
__device__ __forceinline__ float dpp_in_row(float src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), CTRL, 0xf, 0xf, true));
}
constexpr int kRowShl = 0x100, kRowShr = 0x110;

// PASS 1: per-row running (max, sum) partials.  PASS 2: probabilities,
// column sums and diagonal partials.
// grid (key ranges, B*Hq): one work-group per 1024 consecutive keys of one
// query head; the ranges of a head are dispatched in order.  Each wave walks
// its 256 keys in 8 steps of 32; the keys of the next step are loaded while
// the current step is computed.
//
// Diagonal sums in registers (pass 2): in a 16x16 product tile, lane (c, g)
// holds p(row c, key 4g + i), i = 0..3, and lanes 16g .. 16g + 15 form one
// DPP row.  Shifting register i by i lanes (lane c reads lane c + i) puts
// p(row c + i, key 4g + i) in lane c: all four share the offset c - 4g, so
// one add chain per tile sums a diagonal piece; the values whose row c + i
// passes 15 (read with the opposite shift by 16 - i) lie on the offset 16
// lower.  With the step and the tile's (row, key) block the offset is
// base + 16 M + c - 4g, and each lane keeps one partial per M (20 of them
// for the wave's 8 steps); at the end the four lanes (one per g) of every
// offset are added in a fixed order through LDS.
template <typename T, int DH, int PASS>
__global__ __launch_bounds__(256) void vs_proxy_kernel(VsParams P) {
  using Ops = ProxyOps<T, DH>;
  constexpr int kSteps = kVsWaveKeys / 32;
  constexpr int kM = 2 * kSteps + 4;        // diagonal partials per lane
  const int gsz = P.Hq / P.Hkv;
  const int bh = blockIdx.y;
  const int range = blockIdx.x;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n = P.n;
  const int L = min(P.ht.a[h], n);
  const int b = bh / P.Hq;
  const int kv = h / gsz;
  const T* Qb = reinterpret_cast<const T*>(P.Q) + (size_t)bh * n * DH;
  const T* Kb = reinterpret_cast<const T*>(P.K) + ((size_t)b * P.Hkv + kv) * n * DH;
  const int slot = range * 4 + wave;
  const int J0 = slot * kVsWaveKeys;
  const int J1 = min(J0 + kVsWaveKeys, n);
  const int row_base = n - L;    // sampled row r is query n - L + r (valid for r < L)

  typename Ops::QOp q[4][Ops::KS];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int r = 16 * nb + r16;
    if (r < L) Ops::load_k(Qb, row_base + r, g, q[nb]);
    else Ops::zero(q[nb]);
  }

  float m_run[4], l_run[4], lse2[4];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) { m_run[nb] = kNegInf; l_run[nb] = 0.f; lse2[nb] = 0.f; }
  float* cdst = P.vert_score ? P.vert_score : reinterpret_cast<float*>(P.ws_base + P.ws.cbuf);
  cdst += (size_t)bh * n;
  float dacc[kM];
  #pragma unroll
  for (int i = 0; i < kM; ++i) dacc[i] = 0.f;
  if constexpr (PASS == 2) {
    const float* l2 = reinterpret_cast<const float*>(P.ws_base + P.ws.lse2) + (size_t)bh * 64;
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) lse2[nb] = l2[16 * nb + r16];
  }

  typename Ops::QOp kop[2][2][Ops::KS];
  #pragma unroll
  for (int hh = 0; hh < 2; ++hh) Ops::load_k(Kb, min(J0 + 16 * hh + r16, n - 1), g, kop[0][hh]);
  #pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int j = J0 + 32 * step;
    if (j >= J1) break;
    auto& kc = kop[step & 1];
    if (step + 1 < kSteps) {
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) Ops::load_k(Kb, min(j + 32 + 16 * hh + r16, n - 1), g, kop[(step + 1) & 1][hh]);
    }
    floatx4 s[2][4];
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) s[hh][nb] = Ops::dot(kc[hh], q[nb]);
    // valid pairs: sampled row r < L, key < n, key <= query index
    const bool need_mask = (L < 64) || (j + 31 > row_base);
    if (need_mask) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = 16 * nb + r16;
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j + 16 * hh + 4 * g + i;
            if (!(r < L && key < n && key <= row_base + r)) s[hh][nb][i] = kNegInf;
          }
      }
    }
    if constexpr (PASS == 1) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float x = fmaxf(fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), fmaxf(s[0][nb][2], s[0][nb][3])),
                        fmaxf(fmaxf(s[1][nb][0], s[1][nb][1]), fmaxf(s[1][nb][2], s[1][nb][3])));
        x = fmaxf(x, __shfl_xor(x, 16));
        x = fmaxf(x, __shfl_xor(x, 32));
        x *= P.c;
        if (x > m_run[nb]) {
          l_run[nb] *= fast_exp2(m_run[nb] - x);   // m_run = -inf gives 0
          m_run[nb] = x;
        }
        const float msub = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
        float ls = 0.f;
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) ls += fast_exp2(__builtin_fmaf(s[hh][nb][i], P.c, -msub));
        l_run[nb] += ls;
      }
    } else {
      float p[2][4][4];
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) p[hh][nb][i] = fast_exp2(__builtin_fmaf(s[hh][nb][i], P.c, -lse2[nb]));
      // column sums: over the 4 row groups in the lane, then over the 16 lanes of the row group
      float cs[2][4];
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = (p[hh][0][i] + p[hh][1][i]) + (p[hh][2][i] + p[hh][3][i]);
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          x += __shfl_xor(x, 8);
          cs[hh][i] = x;
        }
      // lane r16 < 8 writes key 16*(r16/4) + 4g + r16%4
      if (r16 < 8) {
        const int hh = r16 >> 2, i = r16 & 3;
        float val = 0.f;
        #pragma unroll
        for (int a = 0; a < 2; ++a)
          #pragma unroll
          for (int bq = 0; bq < 4; ++bq)
            if (a == hh && bq == i) val = cs[a][bq];
        const int key = j + 16 * hh + 4 * g + i;
        if (key < n) cdst[key] = val;
      }
      // diagonal pieces of the 8 tiles: tile (nb, hh) has offsets
      // base + 16 (nb - hh - 2 step) + r16 - 4g (M = nb - hh - 2 step) and,
      // for its wrapped values, 16 lower
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float* v = p[hh][nb];
          const float main = v[0] + dpp_in_row<kRowShl + 1>(v[1]) + dpp_in_row<kRowShl + 2>(v[2]) +
                             dpp_in_row<kRowShl + 3>(v[3]);
          const float wrap = dpp_in_row<kRowShr + 15>(v[1]) + dpp_in_row<kRowShr + 14>(v[2]) +
                             dpp_in_row<kRowShr + 13>(v[3]);
          const int M = nb - hh - 2 * step;          // -2*kSteps .. 3
          dacc[M + 2 * kSteps] += main;
          dacc[M - 1 + 2 * kSteps] += wrap;
        }
    }
  }

  if constexpr (PASS == 1) {
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      l_run[nb] += __shfl_xor(l_run[nb], 16);
      l_run[nb] += __shfl_xor(l_run[nb], 32);
    }
    if (g == 0) {
      float* pm = reinterpret_cast<float*>(P.ws_base + P.ws.part_m) + (size_t)bh * 64 * P.ws.nslots;
      float* pl = reinterpret_cast<float*>(P.ws_base + P.ws.part_l) + (size_t)bh * 64 * P.ws.nslots;
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = 16 * nb + r16;
        pm[(size_t)r * P.ws.nslots + slot] = m_run[nb];
        pl[(size_t)r * P.ws.nslots + slot] = l_run[nb];
      }
    }
  } else {
    // slot t of the wave's kVsDiagSlots partials is offset
    // row_base - J0 - (kVsWaveKeys - 1) + t; lane (c, g) holds offset
    // row_base - J0 + 16 M + c - 4g in dacc[M + 2 kSteps]
    __shared__ float part[4][kM][64];
    #pragma unroll
    for (int i = 0; i < kM; ++i) part[wave][i][lane] = dacc[i];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float* dp = reinterpret_cast<float*>(P.ws_base + P.ws.dpart) + ((size_t)bh * P.ws.nslots + slot) * kVsDiagSlots;
    #pragma unroll
    for (int qd = 0; qd < kVsDiagSlots / 64; ++qd) {
      const int t = lane + 64 * qd;
      float acc = 0.f;
      #pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int v = t - (kVsWaveKeys - 1) + 4 * gg;      // 16 M + c
        const int M = (v + 16 * 2 * kSteps) / 16 - 2 * kSteps;   // floor(v / 16), v >= -16 * 2 kSteps
        const int c = v & 15;
        const int mi = M + 2 * kSteps;
        if (mi >= 0 && mi < kM) acc += part[wave][mi][c + 16 * gg];
      }
      dp[t] = acc;
    }
  }
}

// LSE of every sampled row from the per-wave partials: one wave per row,
// lane l folds the partials l, l+64, ... (a fixed order), then the lanes are
// combined by a fixed butterfly.
__global__ __launch_bounds__(256) void vs_lse_kernel(VsParams P, int nslots_used) {
  const int bh = blockIdx.y;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const float* pm = reinterpret_cast<const float*>(P.ws_base + P.ws.part_m) + ((size_t)bh * 64 + r) * P.ws.nslots;
  const float* pl = reinterpret_cast<const float*>(P.ws_base + P.ws.part_l) + ((size_t)bh * 64 + r) * P.ws.nslots;
  float M = kNegInf;
  for (int s = lane; s < nslots_used; s += 64) M = fmaxf(M, pm[s]);
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float Lsum = 0.f;
  if (M != kNegInf)
    for (int s = lane; s < nslots_used; s += 64) Lsum += fast_exp2(pm[s] - M) * pl[s];
  #pragma unroll
  for (int off = 32; off > 0; off >>= 1) Lsum += __shfl_xor(Lsum, off);
  if (lane == 0) {
    float* l2 = reinterpret_cast<float*>(P.ws_base + P.ws.lse2) + (size_t)bh * 64;
    // rows without any key (r >= L) get +inf so that their probabilities are 0
    l2[r] = (Lsum > 0.f) ? M + __log2f(Lsum) : __builtin_huge_valf();
  }
}

// r_d = sum of the (at most two) wave partials whose keys can form offset d.
__global__ __launch_bounds__(256) void vs_diag_kernel(VsParams P) {
  const int bh = blockIdx.y;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const int n = P.n;
  const int L = min(P.ht.a[h], n);
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= n) return;
  const float* dp = reinterpret_cast<const float*>(P.ws_base + P.ws.dpart) + (size_t)bh * P.ws.nslots * kVsDiagSlots;
  const int jlo = max(0, n - L - d), jhi = n - 1 - d;
  const int w1 = jlo / kVsWaveKeys, w2 = jhi / kVsWaveKeys;
  float acc = 0.f;
  for (int w = w1; w <= w2; ++w) {
    const int dbase = n - L - w * kVsWaveKeys - (kVsWaveKeys - 1);
    acc += dp[(size_t)w * kVsDiagSlots + (d - dbase)];
  }
  float* rdst = P.slash_score ? P.slash_score : reinterpret_cast<float*>(P.ws_base + P.ws.rbuf);
  rdst[(size_t)bh * n + d] = acc;
}

// Values exchanged between work-groups of the fused proxy (partials, LSE,
// counters, flags) are read and written with agent-scope atomic loads and
// stores: they bypass the per-XCD L2, which is not coherent across XCDs, so
// no cache-wide write-back or invalidate is needed; a store is complete
// (visible to the whole GPU) once the issuing wave's memory counter drains.
__device__ __forceinline__ void put_c(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<int*>(p), __float_as_int(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_c(const float* p) {
  return __int_as_float(
      __hip_atomic_load(reinterpret_cast<const int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Wait until this wave's memory operations have completed.  The hand-offs
// between work-groups rest on two properties of this hardware rather than
// on release/acquire atomics (which at agent scope write back or invalidate
// the XCD's whole L2 at every hand-off): a store is visible to every XCD
// once the issuing wave's counter has drained, because the exchanged values
// bypass L2; and a wave's loads issue in program order after the flag load
// that released them.  The compiler fences keep the compiler itself from
// moving memory accesses across the wait.
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- single-launch proxy
// The same proxy in one launch (minf_vs_index_fused): pass 1, the LSE fold
// and pass 2 run in one grid, a pass 2 work-group waiting for its head's
// LSE.  Same results up to the summation order of the LSE and slash sums.
// One task: the kVsGroupKeys consecutive keys of key range `range` of VS head
// bh, four waves of kVsWaveKeys keys each.
// PASS 1: running (max, sum) of the sampled rows per wave, combined into one
// partial per work-group.
// PASS 2: exact probabilities; each wave writes the column sums of its keys
// and the complete slash sums of its kVsWaveKeys home offsets, the offsets d whose
// largest key n - 1 - d lies in the wave's keys (their other keys lie at most
// 63 below, which the wave also scores), so every offset is summed by one
// wave in a fixed order.
template <typename T, int DH, int PASS>
__device__ __forceinline__ void fused_task(const VsParams& P, int bh, int range, float (*ptile)[33],
                                           float (*red)[4][64], float* dacc) {
  using Ops = ProxyOps<T, DH>;
  const int gsz = P.Hq / P.Hkv;
  const int h = bh % P.Hq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n = P.n;
  const int L = min(P.ht.a[h], n);
  const int b = bh / P.Hq;
  const int kv = h / gsz;
  const T* Qb = reinterpret_cast<const T*>(P.Q) + (size_t)bh * n * DH;
  const T* Kb = reinterpret_cast<const T*>(P.K) + ((size_t)b * P.Hkv + kv) * n * DH;
  const int J0 = (range * 4 + wave) * kVsWaveKeys;
  if (PASS == 2 && J0 >= n) return;
  const int J1 = min(J0 + kVsWaveKeys, n);
  const int row_base = n - L;    // sampled row r is query n - L + r (valid for r < L)

  typename Ops::QOp q[4][Ops::KS];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int r = 16 * nb + r16;
    if (r < L) Ops::load_k(Qb, row_base + r, g, q[nb]);
    else Ops::zero(q[nb]);
  }

  float m_run[4], l_run[4], lse2[4];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) { m_run[nb] = kNegInf; l_run[nb] = 0.f; lse2[nb] = 0.f; }
  float* cdst = P.vert_score ? P.vert_score : reinterpret_cast<float*>(P.ws_base + P.ws.cbuf);
  cdst += (size_t)bh * n;
  if constexpr (PASS == 2) {
    #pragma unroll
    for (int qd = 0; qd < kVsWaveKeys / 64; ++qd) dacc[lane + 64 * qd] = 0.f;
  }
  if constexpr (PASS == 2) {
    const float* l2 = reinterpret_cast<const float*>(P.ws_base + P.ws.lse2) + (size_t)bh * 64;
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) lse2[nb] = get_c(l2 + 16 * nb + r16);
  }

  // pass 2 also scores the 64 keys below the range: they complete the slash
  // sums of the wave's home offsets (columns are written for j >= J0 only)
  // the keys of the next step are loaded while this step is computed
  const int jbeg = PASS == 2 ? max(0, J0 - 64) : J0;
  typename Ops::QOp kop[2][Ops::KS];
  #pragma unroll
  for (int hh = 0; hh < 2; ++hh) Ops::load_k(Kb, min(jbeg + 16 * hh + r16, n - 1), g, kop[hh]);
  for (int j = jbeg; j < J1; j += 32) {
    typename Ops::QOp knext[2][Ops::KS];
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) Ops::load_k(Kb, min(j + 32 + 16 * hh + r16, n - 1), g, knext[hh]);
    floatx4 s[2][4];
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) s[hh][nb] = Ops::dot(kop[hh], q[nb]);
    // valid pairs: sampled row r < L, key < n, key <= query index
    const bool need_mask = (L < 64) || (j + 31 > row_base);
    if (need_mask) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = 16 * nb + r16;
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j + 16 * hh + 4 * g + i;
            if (!(r < L && key < n && key <= row_base + r)) s[hh][nb][i] = kNegInf;
          }
      }
    }
    if constexpr (PASS == 1) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float x = fmaxf(fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), fmaxf(s[0][nb][2], s[0][nb][3])),
                        fmaxf(fmaxf(s[1][nb][0], s[1][nb][1]), fmaxf(s[1][nb][2], s[1][nb][3])));
        x = fmaxf(x, __shfl_xor(x, 16));
        x = fmaxf(x, __shfl_xor(x, 32));
        x *= P.c;
        if (x > m_run[nb]) {
          l_run[nb] *= fast_exp2(m_run[nb] - x);   // m_run = -inf gives 0
          m_run[nb] = x;
        }
        const float msub = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
        float ls = 0.f;
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) ls += fast_exp2(__builtin_fmaf(s[hh][nb][i], P.c, -msub));
        l_run[nb] += ls;
      }
    } else {
      // probabilities in place of the scores
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) s[hh][nb][i] = fast_exp2(__builtin_fmaf(s[hh][nb][i], P.c, -lse2[nb]));
      // column sums: over the 4 row groups in the lane, then over the 16 lanes of the row group
      float cs[2][4];
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = (s[hh][0][i] + s[hh][1][i]) + (s[hh][2][i] + s[hh][3][i]);
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          x += __shfl_xor(x, 8);
          cs[hh][i] = x;
        }
      // lane r16 < 8 writes key 16*(r16/4) + 4g + r16%4
      if (r16 < 8 && j >= J0) {
        const int hh = r16 >> 2, i = r16 & 3;
        float val = 0.f;
        #pragma unroll
        for (int a = 0; a < 2; ++a)
          #pragma unroll
          for (int bq = 0; bq < 4; ++bq)
            if (a == hh && bq == i) val = cs[a][bq];
        const int key = j + 16 * hh + 4 * g + i;
        if (key < n) cdst[key] = val;
      }
      // diagonal partials: tile[r][jl] = p(row r, key j + jl)
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) ptile[16 * nb + r16][16 * hh + 4 * g + i] = s[hh][nb][i];
      // the tile is private to this wave: LDS accesses of one wave complete in
      // issue order, so a wave-scope fence (no work-group barrier: waves of a
      // group may run different trip counts) orders the writes before the reads
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // the tile's 95 diagonals c = r - jl in [-31, 63], 32 elements per lane:
      // lane l sums c1 = l - 31 and, for l < 31, c2 = l + 33, rows ascending
      float s1 = 0.f, s2 = 0.f;
      #pragma unroll 8
      for (int k = 0; k < 32; ++k) {
        const bool first = lane >= 31 || k <= lane;
        const int r = lane >= 31 ? lane - 31 + k : (k <= lane ? k : k + 32);
        const int jl = lane >= 31 ? k : (k <= lane ? k + 31 - lane : k - lane - 1);
        const float v = ptile[r][jl];
        if (first) s1 += v; else s2 += v;
      }
      // home slot t (offset d = n - kVsWaveKeys - J0 + t) lies on c = base + t here
      const int base = L - kVsWaveKeys + (j - J0);
      const int t1 = lane - 31 - base, t2 = lane + 33 - base;
      if (t1 >= 0 && t1 < kVsWaveKeys) dacc[t1] += s1;
      if (lane < 31 && t2 >= 0 && t2 < kVsWaveKeys) dacc[t2] += s2;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      #pragma unroll
      for (int k = 0; k < Ops::KS; ++k) kop[hh][k] = knext[hh][k];
  }

  if constexpr (PASS == 1) {
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      l_run[nb] += __shfl_xor(l_run[nb], 16);
      l_run[nb] += __shfl_xor(l_run[nb], 32);
    }
    // the four waves' partials are combined in wave order: one (max, sum)
    // per row and work-group
    if (g == 0) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        red[0][wave][16 * nb + r16] = m_run[nb];
        red[1][wave][16 * nb + r16] = l_run[nb];
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int r = threadIdx.x;
      float M = red[0][0][r];
      #pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, red[0][w][r]);
      float S = 0.f;
      if (M != kNegInf) {
        #pragma unroll
        for (int w = 0; w < 4; ++w) S += red[1][w][r] * fast_exp2(red[0][w][r] - M);
      }
      float* pm = reinterpret_cast<float*>(P.ws_base + P.ws.part_m) + (size_t)bh * 64 * P.ws.nslots;
      float* pl = reinterpret_cast<float*>(P.ws_base + P.ws.part_l) + (size_t)bh * 64 * P.ws.nslots;
      put_c(pm + (size_t)r * P.ws.nslots + range, M);
      put_c(pl + (size_t)r * P.ws.nslots + range, S);
    }
  } else {
    float* rdst = P.slash_score ? P.slash_score : reinterpret_cast<float*>(P.ws_base + P.ws.rbuf);
    rdst += (size_t)bh * n;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    #pragma unroll
    for (int qd = 0; qd < kVsWaveKeys / 64; ++qd) {
      const int d = n - kVsWaveKeys - J0 + lane + 64 * qd;
      if (d >= 0) rdst[d] = dacc[lane + 64 * qd];
    }
  }
}

// LSE of the 64 sampled rows of head bh from its per-work-group partials:
// thread (row r, quarter q) takes slots q, q+4, ...; the row maximum first
// (exact in any order), then the rescaled sums in slot order, the quarters
// added by a fixed butterfly (each step commutative, so the four lanes agree).
__device__ __forceinline__ void fused_fold(const VsParams& P, int bh, int nslots_used) {
  const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
  const float* pm = reinterpret_cast<const float*>(P.ws_base + P.ws.part_m) + ((size_t)bh * 64 + r) * P.ws.nslots;
  const float* pl = reinterpret_cast<const float*>(P.ws_base + P.ws.part_l) + ((size_t)bh * 64 + r) * P.ws.nslots;
  float M = kNegInf;
  #pragma unroll 8
  for (int s = q; s < nslots_used; s += 4) M = fmaxf(M, get_c(pm + s));
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  float S = 0.f;
  if (M != kNegInf) {
    #pragma unroll 8
    for (int s = q; s < nslots_used; s += 4) S += get_c(pl + s) * fast_exp2(get_c(pm + s) - M);
  }
  S += __shfl_xor(S, 1);
  S += __shfl_xor(S, 2);
  if (q == 0) {
    float* l2 = reinterpret_cast<float*>(P.ws_base + P.ws.lse2) + (size_t)bh * 64;
    // rows without any key (r >= L) get +inf so that their probabilities are 0
    put_c(l2 + r, (S > 0.f) ? M + __log2f(S) : __builtin_huge_valf());
  }
}

// The work order of the fused proxy launch, built on the host from the head
// table.  Tasks are (batch b, VS head v, key range); idx = b * nvs * nwg +
// first[v] * nwg + range * cnt[v] + (v - first[v]) lists the VS heads of one
// KV group range by range, so they read the same keys one after another.
// Ticket t (the order in which work-groups start) maps to pass 1 task t for
// t < D, then alternates pass 1 task D + k and pass 2 task k, then the last
// pass 2 tasks.  D >= (largest group) * nwg, so a pass 2 task starts after
// every pass 1 task of its head has started.
struct VsFusedMeta {
  int32_t* sync;        // [0] ticket, [1 + i] pass 1 tasks done, [1 + BV + i] LSE ready (i = b * nvs + v)
  int32_t nvs, nwg, T, D;
  uint8_t head[MINF_MAX_HEADS];    // VS heads in ascending order
  uint8_t first[MINF_MAX_HEADS];   // per VS index: first VS index of its KV group
  uint8_t cnt[MINF_MAX_HEADS];     // per VS index: VS heads in its KV group
};

// Polls of a pass 2 task for its head's LSE (about a second): the work order
// makes the wait end (every pass 1 task it waits for started earlier and
// waits for nothing), the bound only keeps a broken order from hanging.
constexpr int kVsWaitPolls = 1 << 22;

// The whole proxy in one launch: pass 1 of a head's key ranges, the LSE fold
// by the last of them to finish, and pass 2, which waits (bounded) for that
// head's LSE.  With the order above, the pass 2 reads of a KV group's keys
// follow its pass 1 reads closely, while they are still in the on-die cache.
template <typename T, int DH>
__global__ __launch_bounds__(256) void vs_fused_kernel(VsParams P, VsFusedMeta M) {
  __shared__ float ptile[4][64][33];
  __shared__ float red[2][4][64];
  __shared__ float dacc[4][kVsWaveKeys];
  __shared__ int s_val;
  if (threadIdx.x == 0) s_val = __hip_atomic_fetch_add(M.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = s_val;
  __syncthreads();
  const int NT = M.T, D = M.D, mid = NT - D;
  int pass, idx;
  if (t < D) { pass = 1; idx = t; }
  else if (t - D < 2 * mid) {
    const int k = t - D;
    pass = (k & 1) ? 2 : 1;
    idx = (k & 1) ? (k >> 1) : D + (k >> 1);
  } else { pass = 2; idx = t - D - mid; }
  if (idx >= NT) return;
  const int per_b = M.nvs * M.nwg;
  const int b = idx / per_b, rem = idx - b * per_b;
  const int v0 = rem / M.nwg;
  const int f = M.first[v0], c = M.cnt[v0];
  const int local = rem - f * M.nwg;
  const int range = local / c, v = f + (local - range * c);
  const int bh = b * P.Hq + M.head[v];
  const int hv = b * M.nvs + v;
  int32_t* done = M.sync + 1;
  int32_t* ready = M.sync + 1 + P.B * M.nvs;
  const int wave = threadIdx.x >> 6;
  if (pass == 1) {
    fused_task<T, DH, 1>(P, bh, range, ptile[wave], red, dacc[wave]);
    drain();
    __syncthreads();
    if (threadIdx.x == 0)
      s_val = __hip_atomic_fetch_add(done + hv, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == M.nwg - 1;
    __syncthreads();
    if (s_val) {
      fused_fold(P, bh, M.nwg);
      drain();
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(ready + hv, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    if (threadIdx.x == 0) {
      int ok = 0;
      for (int i = 0; i < kVsWaitPolls; ++i) {
        if (__hip_atomic_load(ready + hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ok = 1; break; }
        __builtin_amdgcn_s_sleep(8);
      }
      s_val = ok;
      // the LSE loads below stay after the flag load
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    __syncthreads();
    if (!s_val) {
      // the wait ran out (the work order rules this out): report it in the
      // caller's status word and leave defined (zero) column and slash sums
      // for this range rather than unwritten ones
      float* cdst = (P.vert_score ? P.vert_score : reinterpret_cast<float*>(P.ws_base + P.ws.cbuf)) + (size_t)bh * P.n;
      float* rdst = (P.slash_score ? P.slash_score : reinterpret_cast<float*>(P.ws_base + P.ws.rbuf)) + (size_t)bh * P.n;
      const int j0 = range * kVsGroupKeys, j1 = min(j0 + kVsGroupKeys, P.n);
      for (int j = j0 + (int)threadIdx.x; j < j1; j += 256) {
        cdst[j] = 0.f;
        rdst[P.n - 1 - j] = 0.f;     // offset d is home to the range holding key n - 1 - d
      }
      if (threadIdx.x == 0) atomicOr(P.status, (int)MINF_DEV_WAIT_EXHAUSTED);
      return;
    }
    fused_task<T, DH, 2>(P, bh, range, ptile[wave], red, dacc[wave]);
  }
}

// Top-v columns / top-s offsets (selection order: score descending, index
// ascending; outputs ascending), the same radix select as topk.h spread over
// kTopkSeg-element segments of each array: array a = 2 * bh + which (which
// 0: c -> vert_idx, 1: r -> slash_idx).  Per array the workspace holds the
// select state {prefix, mask, remaining}, 256 bins per segment and
// per-segment (greater, equal) counts; kernel boundaries order the passes.
struct TkArray {
  const float* src;
  int32_t* out;
  int k, cap;
  bool vs;
};
__device__ __forceinline__ TkArray tk_array(const VsParams& P, int a) {
  const int bh = a >> 1, which = a & 1;
  const int h = bh % P.Hq;
  TkArray t;
  t.vs = P.ht.kind[h] == MINF_VSLASH;
  if (which == 0) {
    t.src = (P.vert_score ? P.vert_score : reinterpret_cast<const float*>(P.ws_base + P.ws.cbuf)) + (size_t)bh * P.n;
    t.out = P.vert_idx + (size_t)bh * P.max_v;
    t.k = min(P.ht.b[h], P.n);
    t.cap = (int)P.max_v;
  } else {
    t.src = (P.slash_score ? P.slash_score : reinterpret_cast<const float*>(P.ws_base + P.ws.rbuf)) + (size_t)bh * P.n;
    t.out = P.slash_idx + (size_t)bh * P.max_s;
    t.k = min(P.ht.c[h], P.n);
    t.cap = (int)P.max_s;
  }
  return t;
}

// The select state of one array: slot s (s = 0..4) holds (prefix, mask,
// remaining) after s radix digits; slot 0 is the start, slot 4 the k-th key
// T (prefix) and the number of elements equal to T that are taken.  Digit s
// is counted into its own 256-bin histogram (4 per array), to which every
// segment adds its counts with integer atomics (the sums do not depend on
// their order).  The digit of pass s is picked at the start of the next
// launch, by every work-group of it from the same counts, so no launch does
// the picking alone.
__device__ __forceinline__ int32_t* tk_slot(const VsParams& P, int a, int s) {
  return reinterpret_cast<int32_t*>(P.ws_base + P.ws.tk_state) + 4 * (kTkSlots * a + s);
}
__device__ __forceinline__ int32_t* tk_hist(const VsParams& P, int a, int s) {
  return reinterpret_cast<int32_t*>(P.ws_base + P.ws.tk_hist) + 256 * (4 * a + s);
}

// The state after digit s (s = 0..3, at shift 24 - 8 s): from the state
// before it (slot s) and the digit's histogram; every thread of the
// work-group receives it.  Work-group 0 of the launch also stores it in
// slot s + 1.
__device__ void tk_pick(const VsParams& P, int a, int s, bool store, uint32_t* prefix, uint32_t* mask, int* rem) {
  __shared__ int scan[17];
  __shared__ uint32_t n_prefix, n_mask;
  __shared__ int n_rem;
  const int32_t* st = tk_slot(P, a, s);
  const int tot = tk_hist(P, a, s)[threadIdx.x];
  pick_digit(tot, st[2], (uint32_t)st[0], (uint32_t)st[1], 24 - 8 * s, scan, &n_prefix, &n_mask, &n_rem);
  *prefix = n_prefix;
  *mask = n_mask;
  *rem = n_rem;
  if (store && threadIdx.x == 0) {
    int32_t* nx = tk_slot(P, a, s + 1);
    nx[0] = (int32_t)n_prefix;
    nx[1] = (int32_t)n_mask;
    nx[2] = n_rem;
  }
}

// grid (2 * B * Hq): the start state of every array, and its four digit
// histograms cleared
__global__ __launch_bounds__(256) void vs_tk_init_kernel(VsParams P) {
  const int a = blockIdx.x;
  const TkArray t = tk_array(P, a);
  if (!t.vs) return;
  int32_t* h = tk_hist(P, a, 0);
  for (int i = threadIdx.x; i < 4 * 256; i += 256) h[i] = 0;
  if (threadIdx.x != 0) return;
  int32_t* st = tk_slot(P, a, 0);
  const bool all = t.k >= P.n;           // take every element: T = 0, all are greater or equal
  st[0] = 0;                             // prefix
  st[1] = all ? -1 : 0;                  // mask (all ones when done)
  st[2] = all ? P.n : t.k;               // remaining (elements equal to T that are taken)
}

// grid (segments, 2 * B * Hq): digit s (at shift 24 - 8 s) of the keys of one
// segment that match the state before it, added into the digit's histogram;
// for s > 0 the state is first picked from digit s - 1.
__global__ __launch_bounds__(256) void vs_tk_pass_kernel(VsParams P, int s) {
  const int seg = blockIdx.x, a = blockIdx.y;
  const TkArray t = tk_array(P, a);
  if (!t.vs || t.k <= 0 || t.k >= P.n) return;
  __shared__ int hist[4][256];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int lo = seg * kTopkSeg, hi = min(lo + kTopkSeg, P.n);
  // all of the thread's loads are issued before any is used
  constexpr int E = kTopkSeg / 256;
  float x[E];
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lo + tid + 256 * e;
    x[e] = i < hi ? t.src[i] : 0.f;
  }
  uint32_t prefix = 0, mask = 0;
  int rem = 0;
  if (s > 0) {
    tk_pick(P, a, s - 1, seg == 0, &prefix, &mask, &rem);
  } else {
    const int32_t* st = tk_slot(P, a, 0);
    prefix = (uint32_t)st[0];
    mask = (uint32_t)st[1];
  }
  for (int i = tid; i < 4 * 256; i += 256) hist[i >> 8][i & 255] = 0;
  __syncthreads();
  const int shift = 24 - 8 * s;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t key = order_key(x[e]);
    const bool m = lo + tid + 256 * e < hi && (key & mask) == prefix;
    hist_add(hist[wave], m, (key >> shift) & 255u);
  }
  __syncthreads();
  const int c = hist[0][tid] + hist[1][tid] + hist[2][tid] + hist[3][tid];
  if (c) atomicAdd(tk_hist(P, a, s) + tid, c);
}

// grid (segments, 2 * B * Hq): elements above / equal to the k-th key T
__global__ __launch_bounds__(256) void vs_tk_count_kernel(VsParams P) {
  const int seg = blockIdx.x, a = blockIdx.y;
  const TkArray t = tk_array(P, a);
  if (!t.vs || t.k <= 0) return;
  int32_t* cnt = reinterpret_cast<int32_t*>(P.ws_base + P.ws.tk_cnt) + 2 * ((size_t)a * P.ws.tk_segs + seg);
  // the k-th key: picked from the last digit, or (every element taken) the
  // start state, which work-group 0 copies to the last slot
  uint32_t T = 0, mask = 0;
  int rem = 0;
  if (t.k < P.n) {
    tk_pick(P, a, 3, seg == 0, &T, &mask, &rem);
  } else if (seg == 0 && threadIdx.x == 0) {
    const int32_t* s0 = tk_slot(P, a, 0);
    int32_t* s4 = tk_slot(P, a, 4);
    s4[0] = s0[0];
    s4[1] = s0[1];
    s4[2] = s0[2];
  }
  const int lo = seg * kTopkSeg, hi = min(lo + kTopkSeg, P.n);
  constexpr int E = kTopkSeg / 256;
  float x[E];
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lo + threadIdx.x + 256 * e;
    x[e] = i < hi ? t.src[i] : 0.f;
  }
  int gt = 0, eq = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lo + threadIdx.x + 256 * e < hi) {
      const uint32_t key = order_key(x[e]);
      gt += key > T;
      eq += key == T;
    }
  }
  for (int off = 32; off > 0; off >>= 1) { gt += __shfl_xor(gt, off); eq += __shfl_xor(eq, off); }
  __shared__ int pg[4], pe[4];
  if ((threadIdx.x & 63) == 0) { pg[threadIdx.x >> 6] = gt; pe[threadIdx.x >> 6] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    cnt[0] = pg[0] + pg[1] + pg[2] + pg[3];
    cnt[1] = pe[0] + pe[1] + pe[2] + pe[3];
  }
}

// grid (segments, 2 * B * Hq): ordered compaction of each segment; segment
// s writes after the selections of segments < s, and takes the elements
// equal to T that the earlier segments left of the quota.
__global__ __launch_bounds__(256) void vs_tk_write_kernel(VsParams P) {
  const int seg = blockIdx.x, a = blockIdx.y;
  const TkArray t = tk_array(P, a);
  if (!t.vs) return;
  const int tid = threadIdx.x;
  if (t.k <= 0) {
    if (seg == 0)
      for (int i = tid; i < t.cap; i += 256) t.out[i] = -1;
    return;
  }
  const int32_t* st = tk_slot(P, a, 4);
  const int32_t* cnt = reinterpret_cast<const int32_t*>(P.ws_base + P.ws.tk_cnt) + 2 * (size_t)a * P.ws.tk_segs;
  const uint32_t T = (uint32_t)st[0];
  const int need_eq = st[2];
  __shared__ int base_out, eq_before;
  __shared__ int scan[17];
  if (tid == 0) {
    int bo = 0, eb = 0;
    for (int s2 = 0; s2 < seg; ++s2) {
      const int g = cnt[2 * s2], e = cnt[2 * s2 + 1];
      bo += g + max(0, min(e, need_eq - eb));
      eb += e;
    }
    base_out = bo;
    eq_before = eb;
  }
  __syncthreads();
  constexpr int E = kTopkSeg / 256;        // consecutive elements per thread
  const int lo = seg * kTopkSeg + tid * E;
  float x[E];
  #pragma unroll
  for (int e = 0; e < E; ++e) x[e] = lo + e < P.n ? t.src[lo + e] : 0.f;
  uint32_t key[E];
  int n_gt = 0, n_eq = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = order_key(x[e]);
    if (lo + e < P.n) { n_gt += key[e] > T; n_eq += key[e] == T; }
  }
  int tot;
  const int eq_rank0 = eq_before + block_scan_excl<256>(n_eq, scan, &tot);
  const int take_eq = max(0, min(n_eq, need_eq - eq_rank0));
  int pos = base_out + block_scan_excl<256>(n_gt + take_eq, scan, &tot);
  int eq_seen = 0;
  #pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lo + e < P.n) {
      bool sel = key[e] > T;
      if (!sel && key[e] == T) { sel = eq_seen < take_eq; ++eq_seen; }
      if (sel) t.out[pos++] = lo + e;
    }
  }
  if (seg == 0)
    for (int i = t.k + tid; i < t.cap; i += 256) t.out[i] = -1;
}

hipError_t launch_topk(const VsParams& p, hipStream_t st) {
  const unsigned BH = (unsigned)(p.B * p.Hq);
  const dim3 tkg((unsigned)p.ws.tk_segs, 2 * BH);
  hipLaunchKernelGGL(vs_tk_init_kernel, dim3(2 * BH), dim3(256), 0, st, p);
  for (int s = 0; s < 4; ++s) hipLaunchKernelGGL(vs_tk_pass_kernel, tkg, dim3(256), 0, st, p, s);
  hipLaunchKernelGGL(vs_tk_count_kernel, tkg, dim3(256), 0, st, p);
  hipLaunchKernelGGL(vs_tk_write_kernel, tkg, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_t(const VsParams& p, hipStream_t st) {
  const unsigned BH = (unsigned)(p.B * p.Hq);
  const unsigned nwg = (unsigned)((p.n + kVsGroupKeys - 1) / kVsGroupKeys);
  hipLaunchKernelGGL((vs_proxy_kernel<T, DH, 1>), dim3(nwg, BH), dim3(256), 0, st, p);
  hipLaunchKernelGGL(vs_lse_kernel, dim3(16, BH), dim3(256), 0, st, p, (int)(nwg * 4));
  hipLaunchKernelGGL((vs_proxy_kernel<T, DH, 2>), dim3(nwg, BH), dim3(256), 0, st, p);
  hipLaunchKernelGGL(vs_diag_kernel, dim3((p.n + 255) / 256, BH), dim3(256), 0, st, p);
  return launch_topk(p, st);
}

template <typename T, int DH>
hipError_t launch_fused_t(const VsParams& p, hipStream_t st) {
  VsFusedMeta m{};
  const int gsz = p.Hq / p.Hkv;
  int gmax = 0;
  for (int h = 0; h < p.Hq; ++h)
    if (p.ht.kind[h] == MINF_VSLASH) m.head[m.nvs++] = (uint8_t)h;
  for (int v = 0; v < m.nvs;) {
    int e = v;
    while (e < m.nvs && m.head[e] / gsz == m.head[v] / gsz) ++e;
    for (int u = v; u < e; ++u) { m.first[u] = (uint8_t)v; m.cnt[u] = (uint8_t)(e - v); }
    gmax = std::max(gmax, e - v);
    v = e;
  }
  m.nwg = (p.n + kVsGroupKeys - 1) / kVsGroupKeys;
  m.T = p.B * m.nvs * m.nwg;
  m.D = std::min(m.T, (gmax + 1) * m.nwg);
  m.sync = reinterpret_cast<int32_t*>(p.ws_base + p.ws.sync);
  if (m.T > 0) {
    const hipError_t e = launch_fill_i32(m.sync, 1 + 2 * (int64_t)p.B * m.nvs, 0, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((vs_fused_kernel<T, DH>), dim3((unsigned)(2 * m.T)), dim3(256), 0, st, p, m);
  }
  return launch_topk(p, st);
}

}  // namespace

hipError_t launch_vs_index(const VsParams& p, hipStream_t st) {
  if (p.in_bf16) return p.dh == 128 ? launch_t<uint16_t, 128>(p, st) : launch_t<uint16_t, 64>(p, st);
  return p.dh == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

hipError_t launch_vs_index_fused(const VsParams& p, hipStream_t st) {
  if (p.in_bf16) return p.dh == 128 ? launch_fused_t<uint16_t, 128>(p, st) : launch_fused_t<uint16_t, 64>(p, st);
  return p.dh == 128 ? launch_fused_t<float, 128>(p, st) : launch_fused_t<float, 64>(p, st);
}

}  // namespace minf
