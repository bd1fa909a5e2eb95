// Sparse attention over selected tiles: one kernel for the three pattern kinds.
//
// What it computes (PaperTrace 2.1.2 "MInference", section 1.1 Eq. 2 over the
// candidate set N_h(i), merged tile by tile with the running maximum, sum and
// accumulator of section 3.2 Eq. 7-8; blog-zz7 "LLM模型之MInference" section
// 2.3.3 for the per-kind tile walks):
//   o_i = sum_{j in N_h(i)} exp(s_ij - m_i) v_j / sum_{j in N_h(i)} exp(s_ij - m_i),
//   s_ij = scale * q_i . k_j.
//
// Work decomposition (gfx950):
// * one work-group of 4 waves per (batch, head, 64-row query block u);
// * the block's candidate keys are a sequence of 32-key chunks; wave w takes
//   chunks w, w+4, w+8, ... and keeps its OWN running (max, sum, accumulator)
//   for its share of the keys.  Eq. 7-8 hold for any partition of the keys,
//   so the four partial states are merged once, through LDS, at the end; the
//   waves never synchronise inside the loop and never exchange K/V.
// * each wave holds the 64 query rows in registers and streams its K and V
//   rows straight from global memory (L2/MALL) in the operand layout of the
//   16x16x32 bf16 matrix instruction (16x16x4 for fp32):
//     S^T (32 keys x 64 rows) = K_chunk . Q^T       (A = K rows, B = Q^T)
//     O^T (dh x 64 rows)     += V_chunk^T . P^T     (A = V^T,    B = P^T)
//   S^T leaves lane l holding query row l%16 against keys 4*(l/16)+[0..3] of
//   each 16-key half, which is exactly the B-operand layout P^T needs, so the
//   probabilities never move between lanes.  V^T is formed by an 8x8
//   in-register transpose of each lane's 8 key rows (the output columns are
//   permuted so that every lane reads 16 contiguous bytes of a key row and
//   finally owns 32 contiguous output columns).
// * exclusion: invalid pairs get s = -inf BEFORE the row maximum (section 5.1:
//   causal, padding, expanded-tile and duplicate masks before the max).
//   Chunks that need no mask skip the per-element test.
// * lazy rescaling: the running maximum m is only raised when a chunk's
//   maximum exceeds it by more than 2^8 in the exp2 domain; exp2(s - m) is
//   then at most 256, and o = acc / l stays exact because acc and l always use
//   the same m.
// * work order: blockIdx is remapped so that each of the 8 XCDs walks
//   segments of (8 query blocks x the heads of one KV group), heaviest query
//   blocks first; consecutive items on one XCD share K/V lines in its L2.
#include <type_traits>

#include "kernels.h"

namespace minf {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;


// Lane-level description of one 32-key chunk.
struct ChunkDesc {
  int kstart;            // first key (contiguous chunks)
  int vlo, vhi;          // valid keys (contiguous chunks)
  const int32_t* gp;     // key list (gathered chunks) or nullptr
  int gcnt;              // valid entries of gp
  int gbase;             // gathered keys: gbase - entry (span tails, entries are offsets) when gneg
  bool gneg;
  int win;               // > 0: window lower bound j >= i - win + 1 applies
  bool mask;             // per-element test needed
  bool exact;            // a slash span chunk under exact pairs (slash_tile == 1)
};

template <typename T, int DH>
struct Ops;

// ---------------------------------------------------------------- bf16
template <int DH>
struct Ops<uint16_t, DH> {
  static constexpr int KS = DH / 32;     // k-steps of 32 for Q.K
  static constexpr int NV = DH / 16;     // output columns per lane per row group
  static constexpr int QSTRIDE = DH + 8; // LDS row stride (elements), 16-byte pad
  using KOp = u32x4;
  using VRow = typename std::conditional<(NV == 8), u32x4, u32x2>::type;

  __device__ static __forceinline__ void load_k(const uint16_t* __restrict__ Kb, int key, int g, KOp (&k)[KS]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(Kb + (size_t)key * DH + g * (DH / 4));
    #pragma unroll
    for (int s = 0; s < KS; ++s) k[s] = p[s];
  }
  __device__ static __forceinline__ void load_v(const uint16_t* __restrict__ Vb, int key, int r16, VRow& v) {
    const uint16_t* p = Vb + (size_t)key * DH + r16 * NV;
    if constexpr (NV == 8) v = *reinterpret_cast<const u32x4*>(p);
    else v = *reinterpret_cast<const u32x2*>(p);
  }
  __device__ static __forceinline__ void load_q(const uint16_t* sq, int row, int g, KOp (&q)[KS]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(sq + row * QSTRIDE + g * (DH / 4));
    #pragma unroll
    for (int s = 0; s < KS; ++s) q[s] = p[s];
  }
  __device__ static __forceinline__ floatx4 dot(const KOp (&k)[KS], const KOp (&q)[KS], floatx4 a) {
    #pragma unroll
    for (int s = 0; s < KS; ++s) a = mma_bf16(k[s], q[s], a);
    return a;
  }
  // column mb of the 8 key rows (8x8 transpose of 16-bit values, one byte
  // permute per output dword)
  __device__ static __forceinline__ u32x4 vcol(const VRow (&vr)[8], int mb) {
    const uint32_t sel = (mb & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
    #pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(vr[2 * q + 1][mb >> 1], vr[2 * q][mb >> 1], sel);
    return o;
  }
};

// ---------------------------------------------------------------- fp32
template <int DH>
struct Ops<float, DH> {
  static constexpr int KS = DH / 4;
  static constexpr int NV = DH / 16;
  static constexpr int QSTRIDE = DH + 4;
  using KOp = float;
  struct VRow { float x[NV]; };

  __device__ static __forceinline__ void load_k(const float* __restrict__ Kb, int key, int g, KOp (&k)[KS]) {
    const floatx4* p = reinterpret_cast<const floatx4*>(Kb + (size_t)key * DH + g * (DH / 4));
    #pragma unroll
    for (int s = 0; s < KS / 4; ++s) {
      floatx4 x = p[s];
      k[4 * s] = x[0]; k[4 * s + 1] = x[1]; k[4 * s + 2] = x[2]; k[4 * s + 3] = x[3];
    }
  }
  __device__ static __forceinline__ void load_v(const float* __restrict__ Vb, int key, int r16, VRow& v) {
    const floatx4* p = reinterpret_cast<const floatx4*>(Vb + (size_t)key * DH + r16 * NV);
    #pragma unroll
    for (int s = 0; s < NV / 4; ++s) {
      floatx4 x = p[s];
      v.x[4 * s] = x[0]; v.x[4 * s + 1] = x[1]; v.x[4 * s + 2] = x[2]; v.x[4 * s + 3] = x[3];
    }
  }
  __device__ static __forceinline__ void load_q(const float* sq, int row, int g, KOp (&q)[KS]) {
    const floatx4* p = reinterpret_cast<const floatx4*>(sq + row * QSTRIDE + g * (DH / 4));
    #pragma unroll
    for (int s = 0; s < KS / 4; ++s) {
      floatx4 x = p[s];
      q[4 * s] = x[0]; q[4 * s + 1] = x[1]; q[4 * s + 2] = x[2]; q[4 * s + 3] = x[3];
    }
  }
  __device__ static __forceinline__ floatx4 dot(const KOp (&k)[KS], const KOp (&q)[KS], floatx4 a) {
    #pragma unroll
    for (int s = 0; s < KS; ++s) a = mma_f32(k[s], q[s], a);
    return a;
  }
};

// Key position (0..31) inside a chunk of the e-th key a lane holds for V and
// for its S^T entries: e = 4*half + i  ->  16*half + 4*g + i.
__device__ __forceinline__ int vpos(int g, int e) { return ((e >> 2) << 4) + 4 * g + (e & 3); }

template <typename T, int DH>
__global__ __launch_bounds__(256, 1) void attn_kernel(AttnParams P) {
  using O = Ops<T, DH>;
  constexpr int NV = O::NV;
  constexpr int KS = O::KS;
  const int lane = threadIdx.x & 63;
  // wave index in a scalar register: chunk bookkeeping stays wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // ---- work item (XCD-aware order, see header comment)
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int S = 8 * P.gsz;
  const int seg = (slot / S) * 8 + xcd;
  const int within = slot % S;
  if (seg >= P.n_segs) return;
  const int kvg = seg % P.Hkv;
  const int t2 = seg / P.Hkv;
  const int b = t2 / P.n_utiles;
  const int utile = P.n_utiles - 1 - (t2 % P.n_utiles);
  const int u = utile * 8 + within / P.gsz;
  const int h = kvg * P.gsz + within % P.gsz;
  const SampleView SV = sample_view(P, b);
  if (u >= SV.nq) return;

  const int n = SV.n;
  const int kind = __builtin_amdgcn_readfirstlane(P.ht.kind[h]);
  const int row0 = 64 * u;
  const int64_t hrow = SV.q0 + (int64_t)h * n;     // this head's first row in Q, O and lse
  const int64_t hu = (int64_t)h * SV.nq + u;
  const T* __restrict__ Qb = reinterpret_cast<const T*>(P.Q) + hrow * DH;
  const size_t kvoff = (size_t)(SV.kv0 + (int64_t)kvg * n) * DH;
  const T* __restrict__ Kb = reinterpret_cast<const T*>(P.K) + kvoff;
  const T* __restrict__ Vb = reinterpret_cast<const T*>(P.V) + kvoff;

  extern __shared__ float smem[];

  // ---- Q tile -> LDS (rows >= n are zero); read by all four waves
  {
    T* sq = reinterpret_cast<T*>(smem);
    constexpr int PER_ROW = DH * (int)sizeof(T) / 16;   // 16-byte pieces per row
    for (int i = threadIdx.x; i < 64 * PER_ROW; i += 256) {
      const int r = i / PER_ROW, c = i % PER_ROW;
      const int row = row0 + r;
      u32x4 x = {0, 0, 0, 0};
      if (row < n) x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Qb + (size_t)row * DH) + 16 * c);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(sq + r * O::QSTRIDE) + 16 * c) = x;
    }
  }
  __syncthreads();
  const T* sq = reinterpret_cast<const T*>(smem);

  // ---- chunk counts of this item
  int Ca = 0, Cb = 0, Cf = 0;
  int sink_len = 0, wlo = 0, whi = -1, win = 0, ncols = 0;
  const int32_t* colrow = nullptr;
  const int32_t* blkrow = nullptr;
  const int32_t* clo = nullptr;
  const int32_t* chi = nullptr;
  const int32_t* tx = nullptr;
  if (kind == MINF_ASHAPE) {
    const int gk = P.ht.a[h];
    win = P.ht.b[h];
    sink_len = min(gk, min(row0 + 64, n));
    Ca = (sink_len + 31) >> 5;
    if (win > 0) {
      wlo = max(max(gk, row0 - win + 1), 0);
      whi = min(row0 + 63, n - 1);
      Cb = whi >= wlo ? ((whi - wlo + 32) >> 5) : 0;
    }
  } else if (kind == MINF_VSLASH) {
    // counts are clamped to the capacities so that no list is read past its end
    // whole span chunks, then packed chunks of span tails
    Cf = min((long long)max(SV.chunk_cnt[hu], 0), (long long)SV.max_chunks);
    Ca = Cf + min((long long)max(SV.pk_cnt[hu], 0), (long long)(SV.max_tail >> 5));
    tx = SV.tail_x + (int64_t)h * SV.max_tail;
    ncols = min((long long)max(SV.col_cnt[hu], 0), (long long)SV.max_v);
    Cb = (ncols + 31) >> 5;
    colrow = SV.cols + hu * SV.max_v;
    clo = SV.chunk_lo + (int64_t)h * SV.max_chunks;
    chi = SV.chunk_hi + (int64_t)h * SV.max_chunks;
  } else {
    Ca = 2 * (int)min((long long)max(SV.blk_cnt[hu], 0), (long long)SV.max_kb);
    blkrow = SV.blk_idx + hu * SV.max_kb;
  }
  // all of these are wave-uniform; keep them in scalar registers
  Ca = __builtin_amdgcn_readfirstlane(Ca);
  Cb = __builtin_amdgcn_readfirstlane(Cb);
  Cf = __builtin_amdgcn_readfirstlane(Cf);
  sink_len = __builtin_amdgcn_readfirstlane(sink_len);
  wlo = __builtin_amdgcn_readfirstlane(wlo);
  whi = __builtin_amdgcn_readfirstlane(whi);
  win = __builtin_amdgcn_readfirstlane(win);
  ncols = __builtin_amdgcn_readfirstlane(ncols);
  const int C = Ca + Cb;

  floatx4 acc[4][NV];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    #pragma unroll
    for (int mb = 0; mb < NV; ++mb) acc[nb][mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) { m_run[nb] = kNegInf; l_run[nb] = 0.f; }

  // ---- chunk description (wave-uniform)
  auto describe = [&](int k, ChunkDesc& d) {
    d.gp = nullptr; d.gcnt = 0; d.gbase = 0; d.gneg = false; d.win = 0; d.exact = false;
    if (kind == MINF_ASHAPE) {
      if (k < Ca) {
        d.kstart = 32 * k; d.vlo = 0; d.vhi = sink_len - 1;
      } else {
        d.kstart = wlo + 32 * (k - Ca); d.vlo = wlo; d.vhi = whi; d.win = win;
      }
    } else if (kind == MINF_VSLASH) {
      if (k < Cf) {
        const int lo = clo[k], hi = chi[k];
        d.kstart = row0 - hi; d.vlo = max(0, d.kstart); d.vhi = min(row0 - lo, n - 1);
        d.exact = P.slash_tile == 1;
      } else if (k < Ca) {
        // 32 listed tail offsets x: keys 64u - x (padding entries fall below 0)
        d.gp = tx + 32 * (k - Cf); d.gcnt = 32; d.gneg = true; d.gbase = row0;
        d.kstart = 0; d.vlo = 0; d.vhi = n - 1;
      } else {
        const int kk = k - Ca;
        d.gp = colrow + 32 * kk; d.gcnt = min(32, ncols - 32 * kk);
        d.kstart = 0; d.vlo = 0; d.vhi = n - 1;   // validity of listed keys is per position
      }
    } else {
      const int vb = blkrow[k >> 1];
      d.kstart = 64 * vb + 32 * (k & 1); d.vlo = d.kstart; d.vhi = min(d.kstart + 31, n - 1);
      if (vb < 0 || vb > u) { d.kstart = 0; d.vlo = 1; d.vhi = 0; }   // not a causal block: keep nothing
    }
    if (d.gp) {
      d.mask = true;
    } else {
      // a chunk owns exactly its keys [kstart, kstart+31] (its load base may be
      // shifted to stay inside [0, n), so the range must be clipped here)
      d.vlo = max(d.vlo, d.kstart);
      d.vhi = min(d.vhi, d.kstart + 31);
      d.mask = (d.kstart < d.vlo) || (d.kstart + 31 > d.vhi) || (d.kstart + 31 > row0) ||
               (d.win > 0 && d.kstart < row0 + 63 - d.win + 1) || d.exact;
    }
  };
  // The lane's K-operand rows (positions 16*half + r16) are loaded into k;
  // kv[e] gets the key of position vpos(g, e), or -1 when that position is
  // not a candidate.
  auto fetch = [&](const ChunkDesc& d, typename O::KOp (&k)[2][KS], int (&kv)[8]) {
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int p = 16 * hh + r16;
      int key;
      if (d.gp) {
        key = d.gp[p];                 // lists are padded to a multiple of 32 entries
        key = p < d.gcnt ? (d.gneg ? d.gbase - key : key) : 0;
      } else {
        key = d.kstart + p;
      }
      O::load_k(Kb, min(max(key, 0), n - 1), g, k[hh]);
    }
    #pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = vpos(g, e);
      int key;
      if (d.gp) {
        key = d.gp[p];
        if (d.gneg) key = d.gbase - key;
        key = (p < d.gcnt && key >= 0 && key < n) ? key : -1;
      } else {
        key = d.kstart + p;
        key = (key >= d.vlo && key <= d.vhi) ? key : -1;
      }
      kv[e] = key;
    }
  };

  auto qk = [&](const typename O::KOp (&kop)[2][KS], floatx4 (&s)[2][4]) {
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      typename O::KOp q[KS];
      O::load_q(sq, 16 * nb + r16, g, q);
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh) s[hh][nb] = O::dot(kop[hh], q, floatx4{0.f, 0.f, 0.f, 0.f});
    }
  };
  // masks: key(e) = kb0 + ko[e] is the key of the lane's e-th S^T entry
  // (ko[e] < 0 marks a position that is not a candidate)
  auto apply_mask = [&](floatx4 (&s)[2][4], const ChunkDesc& d, int kb0, const int (&ko)[8]) {
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int row = row0 + 16 * nb + r16;
      const int hi = min(d.vhi, row) - kb0;                       // key - kb0 <= hi
      const int lo = (d.win > 0 ? max(d.vlo, row - d.win + 1) : d.vlo) - kb0;
      #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = ko[e];
        bool keep = o >= lo && o <= hi;
        if (keep && d.exact) {
          // Eq. 5 taken literally: row - key a selected offset, or key a
          // selected column (bitmaps from the tile stage)
          const int key = kb0 + o;
          const int bs = n + kBitsPad - 1 - (row - key), bc = key + kBitsPad;
          const uint32_t* sw = SV.slash_bits + (int64_t)h * SV.bits_words;
          const uint32_t* cw = SV.col_bits + (int64_t)h * SV.bits_words;
          keep = ((sw[bs >> 5] >> (bs & 31)) & 1u) || ((cw[bc >> 5] >> (bc & 31)) & 1u);
        }
        if (!keep) s[e >> 2][nb][e & 3] = kNegInf;
      }
    }
  };
  // online softmax (Eq. 7-8 with lazy rescaling) and O^T += V^T P^T
  auto softmax_pv = [&](floatx4 (&s)[2][4], const typename O::VRow (&vr)[8]) {
    float mx[4];
    bool need = false;
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float x = fmaxf(fmaxf(fmaxf(s[0][nb][0], s[0][nb][1]), fmaxf(s[0][nb][2], s[0][nb][3])),
                      fmaxf(fmaxf(s[1][nb][0], s[1][nb][1]), fmaxf(s[1][nb][2], s[1][nb][3])));
      x = fmaxf(x, __shfl_xor(x, 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      mx[nb] = x * P.c;
      need = need || (mx[nb] > m_run[nb] + kTau);
    }
    if (__any(need)) {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float mn = (mx[nb] > m_run[nb] + kTau) ? mx[nb] : m_run[nb];
        const float alpha = (mn == m_run[nb]) ? 1.f : fast_exp2(m_run[nb] - mn);
        #pragma unroll
        for (int mb = 0; mb < NV; ++mb) acc[nb][mb] *= alpha;
        l_run[nb] *= alpha;
        m_run[nb] = mn;
      }
    }
    // probabilities.  For bf16 inputs P is rounded to bf16 for the P.V
    // product and the row sum l adds the ROUNDED values, so the weights that
    // multiply V are exactly normalised (a single dominant key reproduces its
    // value row exactly).
    float p[2][4][4];
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const float msub = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
      #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        #pragma unroll
        for (int i = 0; i < 4; ++i) p[hh][nb][i] = fast_exp2(__builtin_fmaf(s[hh][nb][i], P.c, -msub));
    }
    if constexpr (sizeof(T) == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      u32x4 pop[4];
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        // packed dwords kept in scalars: bit-casting elements extracted from
        // the u32x4 to bf16x2 was miscompiled (every extract read element 0)
        const uint32_t w0 = pack_bf16(p[0][nb][0], p[0][nb][1]), w1 = pack_bf16(p[0][nb][2], p[0][nb][3]);
        const uint32_t w2 = pack_bf16(p[1][nb][0], p[1][nb][1]), w3 = pack_bf16(p[1][nb][2], p[1][nb][3]);
        pop[nb] = u32x4{w0, w1, w2, w3};
        float ls = l_run[nb];
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, ls, false);
        l_run[nb] = ls;
      }
      #pragma unroll
      for (int mb = 0; mb < NV; ++mb) {
        const u32x4 vop = O::vcol(vr, mb);
        #pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb][mb] = mma_bf16(vop, pop[nb], acc[nb][mb]);
      }
    } else {
      #pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float ls = 0.f;
        #pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          #pragma unroll
          for (int i = 0; i < 4; ++i) ls += p[hh][nb][i];
        l_run[nb] += ls;
      }
      #pragma unroll
      for (int e = 0; e < 8; ++e)
        #pragma unroll
        for (int mb = 0; mb < NV; ++mb)
          #pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[nb][mb] = mma_f32(vr[e].x[mb], p[e >> 2][nb][e & 3], acc[nb][mb]);
    }
  };

  // Contiguous chunks are loaded from a wave-uniform base (the chunk's first
  // key, clamped so that all 32 rows lie inside [0, n)) plus constant per-lane
  // offsets; gathered chunks (packed span tails, vertical columns) and tiny
  // sequences use per-lane key indices.
  int vpos_c[8];
  #pragma unroll
  for (int e = 0; e < 8; ++e) vpos_c[e] = vpos(g, e);
  const int Cfast = (n < 32) ? 0 : (kind == MINF_VSLASH ? Cf : C);
  auto load_base = [&](const ChunkDesc& d) { return min(max(d.kstart, 0), n - 32); };
  auto fast_load_k = [&](int lb, typename O::KOp (&kop)[2][KS]) {
    const T* Kc = Kb + (size_t)lb * DH;
    #pragma unroll
    for (int hh = 0; hh < 2; ++hh) O::load_k(Kc, 16 * hh + r16, g, kop[hh]);
  };
  auto fast_load_v = [&](int lb, typename O::VRow (&vr)[8]) {
    const T* Vc = Vb + (size_t)lb * DH;
    #pragma unroll
    for (int e = 0; e < 8; ++e) O::load_v(Vc, vpos_c[e], r16, vr[e]);
  };

  // ---- main loops over this wave's chunks.  One register set each for K and
  //      V: the next chunk's K rows are requested as soon as the current QK
  //      products have consumed the K registers, and the next V rows as soon
  //      as the PV products have consumed V, so each load has about one
  //      step of work to arrive.
  int k = wave;
  if (k < Cfast) {
    typename O::KOp kop[2][KS];
    typename O::VRow vr[8];
    ChunkDesc d, dn;
    describe(k, d);
    int lb = load_base(d);
    fast_load_k(lb, kop);
    fast_load_v(lb, vr);
    while (true) {
      floatx4 s[2][4];
      qk(kop, s);
      const int kn = k + kWaves;
      const bool more = kn < Cfast;
      int lbn = 0;
      if (more) { describe(kn, dn); lbn = load_base(dn); fast_load_k(lbn, kop); }
      if (d.mask) apply_mask(s, d, lb, vpos_c);
      softmax_pv(s, vr);
      k = kn;
      if (!more) break;
      fast_load_v(lbn, vr);
      d = dn;
      lb = lbn;
    }
  }
  if (k < C) {
    typename O::KOp kop[2][KS];
    typename O::VRow vr[8];
    int kv[8], kvn[8];
    ChunkDesc d, dn;
    describe(k, d);
    fetch(d, kop, kv);
    #pragma unroll
    for (int e = 0; e < 8; ++e) O::load_v(Vb, max(kv[e], 0), r16, vr[e]);
    while (true) {
      floatx4 s[2][4];
      qk(kop, s);
      const int kn = k + kWaves;
      const bool more = kn < C;
      if (more) { describe(kn, dn); fetch(dn, kop, kvn); }
      apply_mask(s, d, 0, kv);
      softmax_pv(s, vr);
      if (!more) break;
      #pragma unroll
      for (int e = 0; e < 8; ++e) O::load_v(Vb, max(kvn[e], 0), r16, vr[e]);
      #pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] = kvn[e];
      d = dn;
      k = kn;
    }
  }
  __syncthreads();   // the Q tile's LDS is reused below

  // ---- merge the four waves' partial states (Eq. 7-8 across key subsets)
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    l_run[nb] += __shfl_xor(l_run[nb], 16);
    l_run[nb] += __shfl_xor(l_run[nb], 32);
  }
  constexpr int RS = DH + 4;   // padded LDS row stride (floats)
  float* sm_m = smem;                       // [4][64]
  float* sm_l = smem + kWaves * 64;         // [4][64]
  float* sm_acc = smem + 2 * kWaves * 64;   // [4][64][RS]
  if (g == 0) {
    #pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      sm_m[wave * 64 + 16 * nb + r16] = m_run[nb];
      sm_l[wave * 64 + 16 * nb + r16] = l_run[nb];
    }
  }
  __syncthreads();
  #pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int r = 16 * nb + r16;
    float M = kNegInf;
    #pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 64 + r]);
    float L = 0.f;
    if (M != kNegInf) {
      #pragma unroll
      for (int w = 0; w < kWaves; ++w) L += fast_exp2(sm_m[w * 64 + r] - M) * sm_l[w * 64 + r];
    }
    const float f = (L > 0.f) ? fast_exp2(m_run[nb] - M) / L : 0.f;
    float* dst = sm_acc + ((size_t)wave * 64 + r) * RS + g * (4 * NV);
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
      #pragma unroll
      for (int m4 = 0; m4 < NV / 4; ++m4) {
        floatx4 x = {acc[nb][4 * m4][i] * f, acc[nb][4 * m4 + 1][i] * f, acc[nb][4 * m4 + 2][i] * f,
                     acc[nb][4 * m4 + 3][i] * f};
        *reinterpret_cast<floatx4*>(dst + NV * i + 4 * m4) = x;
      }
    }
    if (wave == 0 && g == 0 && P.lse) {
      const int row = row0 + r;
      if (row < n) P.lse[hrow + row] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
  }
  __syncthreads();
  constexpr int C4 = DH / 4;
  #pragma unroll
  for (int pass = 0; pass < (64 * C4) / 256; ++pass) {
    const int idx = pass * 256 + threadIdx.x;
    const int r = idx / C4, c4 = idx % C4;
    const int row = row0 + r;
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int w = 0; w < kWaves; ++w) o += *reinterpret_cast<const floatx4*>(sm_acc + ((size_t)w * 64 + r) * RS + 4 * c4);
    if (row < n) {
      const size_t off = (size_t)(hrow + row) * DH + 4 * c4;
      if (P.out_bf16) {
        u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(P.O) + off) = pk;
      } else {
        *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.O) + off) = o;
      }
    }
  }
}

size_t attn_smem_bytes(int dh) { return sizeof(float) * (2 * kWaves * 64 + (size_t)kWaves * 64 * (dh + 4)); }

template <typename T, int DH>
static hipError_t launch_t(const AttnParams& p, hipStream_t st) {
  const int S = 8 * p.gsz;
  const int rounds = (p.n_segs + 7) / 8;
  const unsigned grid = (unsigned)rounds * 8u * (unsigned)S;
  const size_t smem = attn_smem_bytes(DH);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<T, DH>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  timing_mark(st, 0);
  hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(grid), dim3(256), smem, st, p);
  timing_mark(st, 1);
  return hipGetLastError();
}

__global__ void write_samples_kernel(SampleBatch b) {
  // one thread per 8-byte word of the descriptors
  constexpr int W = (int)(sizeof(SampleDesc) / 8);
  static_assert(sizeof(SampleDesc) % 8 == 0, "SampleDesc is a whole number of 8-byte words");
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= b.count * W) return;
  reinterpret_cast<uint64_t*>(b.dst)[i] = reinterpret_cast<const uint64_t*>(b.d)[i];
}

hipError_t launch_write_samples(const SampleBatch& b, hipStream_t st) {
  constexpr int W = (int)(sizeof(SampleDesc) / 8);
  const int words = b.count * W;
  if (words <= 0) return hipSuccess;
  hipLaunchKernelGGL(write_samples_kernel, dim3((words + 255) / 256), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnParams& p, int in_bf16, int dh, hipStream_t st) {
  if (in_bf16) return dh == 128 ? launch_attn_bf16_d128(p, st) : launch_t<uint16_t, 64>(p, st);
  return dh == 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace minf
