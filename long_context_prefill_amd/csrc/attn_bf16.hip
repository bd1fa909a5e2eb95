// Sparse attention for bf16 inputs with head dimension 128: the throughput path.
//
// What it computes is the same as the generic kernel in attn.hip
// (PaperTrace 2.1.2 "MInference", section 1.1 Eq. 2 restricted to the
// candidate set N_h(i), merged chunk by chunk with the running maximum, sum
// and accumulator of section 3.2 Eq. 7-8; invalid pairs are -inf before the
// maximum, section 5.1).  The work decomposition is built for gfx950:
//
// * One work-group of two waves per (batch, head, 64-row query block u).
//   Wave w owns query rows 64u + 32w .. +31 for the whole key list, so no
//   partial states are merged at the end.
// * The block's candidate keys are a sequence of 32-key chunks (sink and
//   window chunks, slash-span chunks, gathered vertical columns, or the two
//   halves of a selected 64-key block).  Each chunk's K and V rows are copied
//   once into LDS with direct global->LDS loads (global_load_lds_dwordx4,
//   16 bytes per lane, gathers included), shared by the two waves, in a
//   two-slot ring: the copy of chunk j+1 is in flight while chunk j is
//   computed.  One barrier per chunk.
// * Products on the 32x32x16 bf16 matrix instruction, fp32 accumulation:
//     S^T (32 keys x 32 rows) = K_chunk . Q^T     A = K rows (LDS), B = Q^T (registers)
//     O^T (128 x 32 rows)    += V_chunk^T . P^T   A = V^T (LDS, transposing read), B = P^T
//   The S^T accumulator leaves lane l holding query row l%32 against keys
//   8a + 4(l/32) + b (a, b = 0..3); keys 16s .. 16s+15 of that set are exactly
//   the B-operand P^T of the s-th 16-key PV step, so the probabilities never
//   move between lanes.  V stays row-major in LDS and the A operand V^T is
//   read with ds_read_b64_tr_b16 (lane i of each 16-lane group receives
//   element i%4 of the 8-byte words of lanes 4r + i/4, r = 0..3).
// * Every lane holds one query row, so the running maximum and sum are one
//   register each.  Rescaling is lazy: the maximum moves only when a chunk's
//   maximum exceeds it by 8 in the exp2 domain (exp2(s - m) <= 256 otherwise),
//   which needs no cross-lane operation on the common path; o = acc / l stays
//   exact because acc and l always use the same m.
// * P is rounded to bf16 for the PV product and the row sum adds the rounded
//   values (v_dot2_f32_bf16), so the weights that multiply V are exactly
//   normalised.
// * LDS layout, per slot: K rows then V rows, 256 bytes each.  The 16-byte
//   piece p of key row r sits at p ^ (r & 15) for K and p ^ 4(r & 3) for V,
//   which keeps the K operand reads (16 consecutive rows, one piece) and the
//   transposing V reads (8 rows, 64 bytes each) free of bank conflicts; the
//   copies write 4 whole rows per instruction.
// * Occupancy: 4 work-groups (8 waves) per CU, two waves per SIMD, so one
//   wave's softmax overlaps the other's matrix products.
#include "kernels.h"

namespace minf {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kDH = 128;
constexpr int kRowB = kDH * 2;          // bytes per K or V row
constexpr int kTileB = 32 * kRowB;      // 8 KiB: one chunk of K (or V)
constexpr int kSlotB = 2 * kTileB;      // K then V
constexpr int kSmem = 2 * kSlotB;       // two slots
constexpr float kTau = 8.0f;
constexpr float kMInit = -1.0e30f;      // running maximum before any key (finite)

__device__ __forceinline__ floatx16 mma32(u32x4 a, u32x4 b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// 16 bytes per lane from global memory (base + voff) into LDS at dst + 16 *
// lane; base and dst are wave-uniform.  Written as inline assembly so that
// the compiler does not treat every later LDS read as dependent on the copy
// (it would wait for the next chunk's copies before reading the current
// slot); completion is waited for explicitly before the barrier of each
// chunk.  M0 carries the LDS address and is restored afterwards; one wait
// state separates the M0 write from the copy.
__device__ __forceinline__ void copy16(const char* base, uint32_t voff, uint32_t dst) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(base), "s"(dst)
      : "memory");
}

__device__ __forceinline__ u32x2 read_tr(const lds_char* p) {
  const short4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Wave-uniform read of an index list through the constant address space, so
// that it becomes a scalar load: vector loads share the counter that the LDS
// copies are waited on with.  The lists are read-only during the kernel.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

struct Chunk {
  int kstart;         // first key of a contiguous chunk
  int vlo, vhi;       // keys kept from a contiguous chunk
  int win;            // > 0: also j >= i - win + 1
  const int32_t* gp;  // key list of a gathered chunk, else nullptr
  int gcnt;           // entries of gp
};

}  // namespace

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_d128_kernel(AttnParams P) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item: each XCD (blockIdx mod 8) walks segments of 8 query
  //      blocks x the query heads of one KV group, heaviest blocks first
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
  if (u >= P.nq) return;

  const int n = P.n;
  const int kind = __builtin_amdgcn_readfirstlane(P.ht.kind[h]);
  const int row0 = 64 * u;
  const int rw0 = row0 + 32 * wave;     // this wave's first row
  const int myrow = rw0 + l32;
  const size_t bh = (size_t)b * P.Hq + h;
  const size_t kvoff = ((size_t)b * P.Hkv + kvg) * (size_t)n * kDH;
  const char* __restrict__ Kb = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(P.K) + kvoff);
  const char* __restrict__ Vb = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(P.V) + kvoff);

  __shared__ __attribute__((aligned(16))) char smem_g[kSmem];
  lds_char* smem = (lds_char*)smem_g;

  // ---- Q^T operand in registers: lane l holds row myrow, 16-byte pieces 2t + hh
  u32x4 q[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(P.Q) +
                                                     (bh * n + min(myrow, n - 1)) * (size_t)kDH);
    #pragma unroll
    for (int t = 0; t < 8; ++t) {
      q[t] = qp[2 * t + hh];
      if (myrow >= n) q[t] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- chunk counts of this item (wave-uniform)
  int Ca = 0, Cb = 0, sink_len = 0, wlo = 0, whi = -1, win = 0, ncols = 0;
  const int32_t* colrow = nullptr;
  const int32_t* blkrow = nullptr;
  const int32_t* clo = nullptr;
  const int32_t* chi = nullptr;
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
    Ca = (int)min((long long)max(ld_uniform(P.chunk_cnt, bh * P.nq + u), 0), (long long)P.max_chunks);
    ncols = (int)min((long long)max(ld_uniform(P.col_cnt, bh * P.nq + u), 0), (long long)P.max_v);
    Cb = (ncols + 31) >> 5;
    colrow = P.cols + (bh * P.nq + u) * P.max_v;
    clo = P.chunk_lo + bh * P.max_chunks;
    chi = P.chunk_hi + bh * P.max_chunks;
  } else {
    Ca = 2 * (int)min((long long)max(ld_uniform(P.blk_cnt, bh * P.nq + u), 0), (long long)P.max_kb);
    blkrow = P.blk_idx + (bh * P.nq + u) * P.max_kb;
  }
  Ca = __builtin_amdgcn_readfirstlane(Ca);
  Cb = __builtin_amdgcn_readfirstlane(Cb);
  sink_len = __builtin_amdgcn_readfirstlane(sink_len);
  wlo = __builtin_amdgcn_readfirstlane(wlo);
  whi = __builtin_amdgcn_readfirstlane(whi);
  win = __builtin_amdgcn_readfirstlane(win);
  ncols = __builtin_amdgcn_readfirstlane(ncols);
  const int C = Ca + Cb;

  auto describe = [&](int k, Chunk& d) {
    d.gp = nullptr; d.gcnt = 0; d.win = 0;
    if (kind == MINF_ASHAPE) {
      if (k < Ca) {
        d.kstart = 32 * k; d.vlo = 0; d.vhi = sink_len - 1;
      } else {
        d.kstart = wlo + 32 * (k - Ca); d.vlo = wlo; d.vhi = whi; d.win = win;
      }
    } else if (kind == MINF_VSLASH) {
      if (k < Ca) {
        const int lo = ld_uniform(clo, k), hi = ld_uniform(chi, k);
        d.kstart = row0 - hi; d.vlo = max(0, d.kstart); d.vhi = min(row0 - lo, n - 1);
      } else {
        const int kk = k - Ca;
        d.gp = colrow + 32 * kk; d.gcnt = min(32, ncols - 32 * kk);
        d.kstart = 0; d.vlo = 0; d.vhi = n - 1;
      }
    } else {
      const int vb = ld_uniform(blkrow, k >> 1);
      d.kstart = 64 * vb + 32 * (k & 1); d.vlo = d.kstart; d.vhi = min(d.kstart + 31, n - 1);
      if (vb < 0 || vb > u) { d.kstart = 0; d.vlo = 1; d.vhi = 0; }   // not a causal block: keep nothing
    }
    if (!d.gp) {
      // a chunk owns exactly its keys [kstart, kstart + 31]
      d.vlo = max(d.vlo, d.kstart);
      d.vhi = min(d.vhi, d.kstart + 31);
    }
  };

  // ---- copy offsets.  Wave w copies rows 16w + 4i + lane/16 (i = 0..3) of
  //      each tile; lane l writes LDS piece l%16 of its row, which holds the
  //      row's piece (l%16) ^ swz(row).
  const int crow0 = 16 * wave + (lane >> 4);
  const int cpiece = lane & 15;
  uint32_t koff[4], voff[4];
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = crow0 + 4 * i;
    koff[i] = (uint32_t)(r * kRowB + 16 * (cpiece ^ (r & 15)));
    voff[i] = (uint32_t)(r * kRowB + 16 * (cpiece ^ (4 * (r & 3))));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](const Chunk& d, int sl) {
    const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_base + sl * kSlotB + 4096 * wave);
    const uint32_t lv = lk + kTileB;
    if (!d.gp && d.kstart >= 0 && d.kstart + 31 < n) {
      const char* kb = Kb + (size_t)d.kstart * kRowB;
      const char* vb = Vb + (size_t)d.kstart * kRowB;
      #pragma unroll
      for (int i = 0; i < 4; ++i) copy16(kb, koff[i], lk + 1024 * i);
      #pragma unroll
      for (int i = 0; i < 4; ++i) copy16(vb, voff[i], lv + 1024 * i);
    } else {
      // per-lane rows: clamped into [0, n) (the excess keys are masked) or
      // gathered from the column list; all keys are read before any copy
      uint32_t rb[4];
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = crow0 + 4 * i;
        int key = d.kstart + r;
        if (d.gp) key = r < d.gcnt ? d.gp[r] : 0;
        rb[i] = (uint32_t)min(max(key, 0), n - 1) * kRowB;
      }
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = crow0 + 4 * i;
        copy16(Kb, rb[i] + 16 * (cpiece ^ (r & 15)), lk + 1024 * i);
        copy16(Vb, rb[i] + 16 * (cpiece ^ (4 * (r & 3))), lv + 1024 * i);
      }
    }
  };

  // ---- operand read offsets
  // K: lane l reads row l%32, piece 2t + hh
  uint32_t kr[8];
  #pragma unroll
  for (int t = 0; t < 8; ++t) kr[t] = (uint32_t)(l32 * kRowB + 16 * ((2 * t + hh) ^ (l32 & 15)));
  // V^T (transposing read): lane 16G + 4r + qq supplies row 16s + 8rho + 4(G/2) + r,
  // columns 32mb + 16(G%2) + 4qq .. +3
  uint32_t vr[4];
  {
    const int G = lane >> 4, r = (lane >> 2) & 3, qq = lane & 3;
    #pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      vr[mb] = (uint32_t)((4 * (G >> 1) + r) * kRowB + 16 * (4 * (mb ^ r) + 2 * (G & 1) + (qq >> 1)) + 8 * (qq & 1));
  }

  floatx16 acc[4];
  #pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    #pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = kMInit, l_run = 0.f;
  const float cfac = P.c;

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // What a chunk needs from this wave (wave-uniform): whether any of its keys
  // survives for the wave's rows, and whether some pair needs the per-element
  // test.  For a gathered chunk that needs the test, gbits gets bit i set when
  // the lane's i-th key (position 8(i/4) + 4hh + i%4) is kept for its row;
  // those keys are loaded here, before the next chunk's copies are in flight.
  struct Plan { bool any, mask; uint32_t gbits; };
  auto plan = [&](const Chunk& d) {
    Plan pl{false, false, 0u};
    if (d.gp) {
      if (d.gcnt <= 0) return pl;
      const int gfirst = ld_uniform(d.gp, 0);
      const int glast = ld_uniform(d.gp, d.gcnt - 1);
      pl.any = gfirst <= rw0 + 31;
      pl.mask = d.gcnt < 32 || glast > rw0;
      if (pl.any && pl.mask) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int pos = 8 * (i >> 2) + 4 * hh + (i & 3);
          const int key = pos < d.gcnt ? d.gp[pos] : n;
          pl.gbits |= (key <= myrow ? 1u : 0u) << i;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    } else {
      const int hi = min(d.vhi, rw0 + 31);
      const int lo = d.win > 0 ? max(d.vlo, rw0 - d.win + 1) : d.vlo;
      pl.any = lo <= hi;
      pl.mask = d.kstart < d.vlo || d.kstart + 31 > d.vhi || d.kstart + 31 > rw0 ||
                (d.win > 0 && d.kstart < rw0 + 31 - d.win + 1);
    }
    return pl;
  };

  auto compute = [&](const Chunk& d, const Plan& pl, int sl) {
    if (!pl.any) return;
    const bool mask = pl.mask;
    const lds_char* ks = smem + sl * kSlotB;
    const lds_char* vs = ks + kTileB;

    floatx16 s;
    #pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    #pragma unroll
    for (int t = 0; t < 8; ++t) s = mma32(*(lds_u32x4*)(ks + kr[t]), q[t], s);

    if (mask) {
      // element i holds key position 8(i/4) + 4hh + i%4 of the chunk
      if (d.gp) {
        #pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((pl.gbits >> i) & 1u)) s[i] = kNegInf;
      } else {
        const int hi = min(d.vhi, myrow) - d.kstart;
        const int lo = (d.win > 0 ? max(d.vlo, myrow - d.win + 1) : d.vlo) - d.kstart;
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int pos = 8 * (i >> 2) + 4 * hh + (i & 3);
          if (!(pos >= lo && pos <= hi)) s[i] = kNegInf;
        }
      }
    }

    // online softmax, lazy rescaling
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    mx *= cfac;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau)) {
      const float pm = fmaxf(mx, __shfl_xor(mx, 32));      // the row's other 16 keys
      const float mn = pm > m_run + kTau ? pm : m_run;
      const float alpha = fast_exp2(m_run - mn);
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    u32x4 pb[2];
    #pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t w[4];
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(__builtin_fmaf(s[8 * st + 2 * e], cfac, -m_run));
        const float p1 = fast_exp2(__builtin_fmaf(s[8 * st + 2 * e + 1], cfac, -m_run));
        w[e] = pack_bf16(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, l_run, false);
      }
      pb[st] = u32x4{w[0], w[1], w[2], w[3]};
    }

    // O^T += V^T P^T
    #pragma unroll
    for (int st = 0; st < 2; ++st) {
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const lds_char* p = vs + vr[mb] + 4096 * st;
        const u32x2 lo = read_tr(p);
        const u32x2 hi2 = read_tr(p + 2048);
        const u32x4 va = {lo[0], lo[1], hi2[0], hi2[1]};
        acc[mb] = mma32(va, pb[st], acc[mb]);
      }
    }
  };

  // ---- main loop: copy chunk j+1 while chunk j is computed
  if (C > 0) {
    Chunk dc, dn;
    describe(0, dc);
    issue(dc, 0);
    for (int j = 0; j < C; ++j) {
      // this wave's copies of chunk j have landed; after the barrier the other
      // wave's have too, and both have finished reading chunk j-1's slot
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const Plan pl = plan(dc);
      if (j + 1 < C) {
        describe(j + 1, dn);
        issue(dn, (j + 1) & 1);
      }
      compute(dc, pl, j & 1);
      dc = dn;
    }
  }

  // ---- finish: the row's sum over both lane halves, O = acc / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float f = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (myrow < n) {
    const size_t obase = (bh * n + myrow) * (size_t)kDH;
    #pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = 32 * mb + 8 * a + 4 * hh;
        const floatx4 o = {acc[mb][4 * a] * f, acc[mb][4 * a + 1] * f, acc[mb][4 * a + 2] * f, acc[mb][4 * a + 3] * f};
        if (P.out_bf16) {
          const u32x2 pk = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(P.O) + obase + col) = pk;
        } else {
          *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.O) + obase + col) = o;
        }
      }
    }
    if (hh == 0 && P.lse)
      P.lse[bh * n + myrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

hipError_t launch_attn_bf16_d128(const AttnParams& p, hipStream_t st) {
  const int S = 8 * p.gsz;
  const int rounds = (p.n_segs + 7) / 8;
  const unsigned grid = (unsigned)rounds * 8u * (unsigned)S;
  hipLaunchKernelGGL(attn_bf16_d128_kernel, dim3(grid), dim3(128), 0, st, p);
  return hipGetLastError();
}

}  // namespace minf
