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
#include <type_traits>

#include "kernels.h"

namespace minf {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const int32_t lds_i32;

constexpr int kDH = 128;
constexpr int kRowB = kDH * 2;          // bytes per K or V row
constexpr int kTileB = 32 * kRowB;      // 8 KiB: one chunk of K (or V)
constexpr int kSlotB = 2 * kTileB;      // K then V
constexpr int kRing = 2 * kSlotB;       // two K/V slots
constexpr int kListB = 32 * 4;          // one gathered chunk's 32 list entries
constexpr int kTicket = kRing + 3 * kListB;  // the next item's queue ticket
constexpr int kSmem = kTicket + 16;          // K/V ring, entry-list ring, ticket
constexpr float kTau = 8.0f;
constexpr float kMInit = -1.0e30f;      // running maximum before any key (finite)

__device__ __forceinline__ floatx16 mma32(u32x4 a, u32x4 b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
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

// A chunk of 32 keys as the pipeline sees it (wave-uniform).
constexpr int kFast = 1;     // keys kstart .. kstart+31, all inside [0, n): one affine copy
constexpr int kMask = 2;     // some pair of this wave's rows needs the per-element test
constexpr int kNone = 4;     // no pair of this wave's rows is kept
constexpr int kGather = 8;   // keys are column-list entries kstart .. kstart+vhi-1
constexpr int kWin = 16;     // an A-shape window chunk: keys j >= i - window + 1 only
constexpr int kExact = 32;   // a slash span chunk under exact pairs (slash_tile == 1)
constexpr int kNeg = 64;     // gathered from the tail list: entries are offsets x, keys 64u - x
struct Chunk {
  int kstart;   // first key (contiguous) or first column-list entry (gathered)
  int vlo, vhi; // contiguous: keys kept within the chunk; gathered: vhi = entries
  int flags;
};

// The chunk lists of one work item (head h of sequence S, query block u): Ca chunks
// of the first list (sink, slash spans or selected blocks) and Cb of the
// second (window or gathered columns).  For Vertical-Slash heads the first
// list is Cf whole 32-offset span chunks followed by Ca - Cf packed chunks of
// span tails (32 listed offsets x each, keys 64u - x).  Shared by the cost pass of the
// scheduler and the attention kernel.
struct ItemLists {
  int Ca, Cb, Cf, sink_len, wlo, whi, win, ncols;
  const int32_t* colrow;
  const int32_t* tx;
  const int32_t* blkrow;
  const int32_t* clo;
  const int32_t* chi;
};

__device__ __forceinline__ ItemLists item_lists(const AttnParams& P, const SampleView& S, int h, int kind, int u) {
  ItemLists L{0, 0, 0, 0, 0, -1, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
  const int n = S.n, row0 = 64 * u;
  const int64_t hu = (int64_t)h * S.nq + u;
  if (kind == MINF_ASHAPE) {
    const int gk = P.ht.a[h];
    L.win = P.ht.b[h];
    L.sink_len = min(gk, min(row0 + 64, n));
    L.Ca = (L.sink_len + 31) >> 5;
    if (L.win > 0) {
      L.wlo = max(max(gk, row0 - L.win + 1), 0);
      L.whi = min(row0 + 63, n - 1);
      L.Cb = L.whi >= L.wlo ? ((L.whi - L.wlo + 32) >> 5) : 0;
    }
  } else if (kind == MINF_VSLASH) {
    // counts are clamped to the capacities so that no list is read past its end
    L.Cf = (int)min((long long)max(ld_uniform(S.chunk_cnt, hu), 0), (long long)S.max_chunks);
    L.Ca = L.Cf + (int)min((long long)max(ld_uniform(S.pk_cnt, hu), 0), (long long)(S.max_tail >> 5));
    // (the stride passes through readfirstlane: without it the compiler
    // kept the tail list's base in vector registers and failed to build the
    // scalar loads of its entries)
    L.tx = S.tail_x + (int64_t)h * __builtin_amdgcn_readfirstlane((int)S.max_tail);
    L.ncols = (int)min((long long)max(ld_uniform(S.col_cnt, hu), 0), (long long)S.max_v);
    L.Cb = (L.ncols + 31) >> 5;
    L.colrow = S.cols + hu * S.max_v;
    L.clo = S.chunk_lo + (int64_t)h * S.max_chunks;
    L.chi = S.chunk_hi + (int64_t)h * S.max_chunks;
  } else {
    L.Ca = 2 * (int)min((long long)max(ld_uniform(S.blk_cnt, hu), 0), (long long)S.max_kb);
    L.blkrow = S.blk_idx + hu * S.max_kb;
  }
  return L;
}

}  // namespace

// ---------------------------------------------------------------- schedule
// Work items are (batch, head, query block) triples, handed out through one
// queue per XCD: the attention kernel runs persistent work-groups (four per
// CU) and work-group i serves the queue of XCD i mod 8, the XCD the
// hardware dispatches it to; once that queue is empty it takes items from
// the other queues in turn, so that the XCDs finish together even where
// their items ran at different speeds.  Items are grouped into units:
// * a Vertical-Slash or A-shape unit is a run of consecutive query blocks of
//   one (batch, head) pair (the run length comes from attn_sched_shape); its
//   blocks are queued from the last to the first;
// * a Block-Sparse unit holds every Block-Sparse head of one (batch, KV
//   group) over such a run, interleaved per query block: heads that share K
//   and V and select nearly the same key blocks run side by side.  Beyond
//   kGroupAllMinN tokens the Vertical-Slash and A-shape heads of a group
//   are grouped the same way (group_kinds).
// Units are costed by their exact chunk counts.  KV groups are taken in
// order, and within a group the units are handed out largest first, eight
// at a time, to the eight XCD queues in ascending order of load, so the
// XCDs work through the groups
// together (the active group's K and V stay in the memory-side cache).  The
// work-groups that run together on one XCD are consecutive query blocks of
// one head (or one KV group), whose key sets largely coincide, so their K/V
// rows are also shared in that XCD's L2.

// Heads of h's KV group with h's pattern kind: their number, and h's rank
// among them.
__device__ __forceinline__ int kind_group(const AttnParams& P, int h, int* rank) {
  const int g0 = (h / P.gsz) * P.gsz, kind = P.ht.kind[h];
  int cnt = 0, r = -1;
  for (int k = g0; k < g0 + P.gsz; ++k) {
    if (P.ht.kind[k] != kind) continue;
    if (k == h) r = cnt;
    ++cnt;
  }
  *rank = r;
  return cnt;
}
// k-th head of the given kind in the KV group that starts at head g0
__device__ __forceinline__ int kind_head(const AttnParams& P, int g0, int k, int kind) {
  for (int j = g0; j < g0 + P.gsz; ++j)
    if (P.ht.kind[j] == kind && k-- == 0) return j;
  return g0;
}
__device__ __forceinline__ bool grouped(const AttnParams& P, int kind) { return (P.group_kinds >> kind) & 1; }
// Items of a unit (0 for the units of grouped heads other than the first of
// their kind in their group, whose items the first head's unit carries).
__device__ __forceinline__ int unit_items(const AttnParams& P, int unit, int* u0, int* u1, int* nbs) {
  const int bhi = unit / P.sched_P, part = unit % P.sched_P;
  const int h = bhi % P.Hq;
  *u0 = part * P.sched_R;
  const int nq = P.samples ? P.samples[bhi / P.Hq].nq : P.nq;   // this sequence's blocks
  *u1 = min(*u0 + P.sched_R, nq);
  *nbs = 1;
  if (*u0 >= *u1) return 0;
  if (grouped(P, P.ht.kind[h])) {
    int r;
    *nbs = kind_group(P, h, &r);
    if (r != 0) return 0;
    return (*u1 - *u0) * *nbs;
  }
  return *u1 - *u0;
}

__global__ __launch_bounds__(256) void attn_cost_kernel(AttnParams P) {
  const int unit = blockIdx.x;
  int u0, u1, nbs;
  const int items = unit_items(P, unit, &u0, &u1, &nbs);
  const int bhi = unit / P.sched_P;
  const int b = bhi / P.Hq, h = bhi % P.Hq;
  const int kind = P.ht.kind[h];
  const SampleView S = sample_view(P, b);
  long long c = 0;
  for (int i = (int)threadIdx.x; i < items; i += 256) {
    const int u = u1 - 1 - i / nbs;
    const int hh = grouped(P, kind) ? kind_head(P, (h / P.gsz) * P.gsz, i % nbs, kind) : h;
    const ItemLists L = item_lists(P, S, hh, kind, u);
    c += L.Ca + L.Cb + 2;   // + fixed cost of an item (Q load, output)
  }
  __shared__ long long sh[256];
  sh[threadIdx.x] = c;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) sh[threadIdx.x] += sh[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) P.sched_cost[unit] = items > 0 ? sh[0] : -1;
}

__global__ __launch_bounds__(256) void attn_sched_kernel(AttnParams P) {
  const int U = P.sched_units;
  const int tid = threadIdx.x, lane = tid & 63;
  // The units of one KV group are contiguous (heads g0 .. g0 + gsz - 1 of one
  // batch entry); rank them by (group ascending, cost descending, unit
  // ascending), comparing within the group only.  Queue order is rank order.
  const int per_group = P.gsz * P.sched_P;
  __shared__ int s_unit[kMaxUnits], s_cost[kMaxUnits], s_items[kMaxUnits];
  const bool staged = U <= kMaxUnits;   // beyond kMaxUnits units: global memory
  for (int u = tid; u < U; u += 256) {
    const long long cu = P.sched_cost[u];
    const int g0 = u - u % per_group;
    int r = g0;
    #pragma unroll 8
    for (int v = g0; v < g0 + per_group; ++v) {
      const long long cv = P.sched_cost[v];
      r += (cv > cu) || (cv == cu && v < u);
    }
    P.sched_order[r] = u;
    if (staged) {
      int u0, u1, nbs;
      s_unit[r] = u;
      s_cost[r] = (int)min(cu, (long long)0x7fffffff);
      s_items[r] = unit_items(P, u, &u0, &u1, &nbs);
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  // Greedy pass on one wave, eight units at a time: lane x < 8 holds XCD
  // x's load and item count; each round of a group hands its next eight
  // units (largest first) to the eight XCDs in ascending order of load
  // (ties to the lower index), the least-loaded XCD taking the largest unit.
  long long myload = 0;
  int mycnt = 0;
  for (int g0 = 0; g0 < U; g0 += per_group) {
    for (int j0 = 0; j0 < per_group; j0 += 8) {
      // this lane's XCD rank by load (readlane with constant lanes: no LDS)
      int rank = 0;
      #pragma unroll
      for (int y = 0; y < 8; ++y) {
        const int lo32 = __builtin_amdgcn_readlane((int)(uint32_t)myload, y);
        const int hi32 = __builtin_amdgcn_readlane((int)(myload >> 32), y);
        const long long ly = ((long long)hi32 << 32) | (uint32_t)lo32;
        rank += (ly < myload) || (ly == myload && y < lane);
      }
      const int j = j0 + rank;
      if (lane < 8 && j < per_group) {
        const int o = g0 + j;
        int unit, items;
        long long cu;
        if (staged) {
          unit = s_unit[o];
          cu = s_cost[o];
          items = s_items[o];
        } else {
          unit = P.sched_order[o];
          cu = P.sched_cost[unit];
          int u0, u1, nbs;
          items = unit_items(P, unit, &u0, &u1, &nbs);
        }
        if (cu < 0) {
          P.unit_xcd[unit] = -1;
        } else {
          P.unit_xcd[unit] = lane;
          P.unit_off[unit] = mycnt;
          mycnt += items;
          myload += cu;
        }
      }
    }
  }
  // queue offsets: exclusive sum of the item counts over lanes 0..7
  int incl = lane < 8 ? mycnt : 0;
  #pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane < 8) {
    P.queue_meta[lane] = incl - mycnt;
    P.queue_meta[8 + lane] = mycnt;
    P.queue_meta[16 + lane] = 0;     // the queue counters start at zero
  }
}

__global__ __launch_bounds__(256) void attn_fill_kernel(AttnParams P) {
  const int unit = blockIdx.x;
  const int x = P.unit_xcd[unit];
  if (x < 0) return;
  int u0, u1, nbs;
  const int items = unit_items(P, unit, &u0, &u1, &nbs);
  const int bhi = unit / P.sched_P;
  const int b = bhi / P.Hq, h = bhi % P.Hq;
  const int kind = P.ht.kind[h];
  const bool grp = grouped(P, kind);
  int32_t* q = P.queue + P.queue_meta[x] + P.unit_off[unit];
  for (int i = (int)threadIdx.x; i < items; i += 256) {
    const int u = u1 - 1 - i / nbs;
    const int hh = grp ? kind_head(P, (h / P.gsz) * P.gsz, i % nbs, kind) : h;
    q[i] = ((b * P.Hq + hh) * P.nq) + u;
  }
}

namespace {

// Copies of one 32-key chunk of K (or V): four copies of 16 bytes per lane
// from global memory (base + voff[i] + 1024 i) into LDS at dst + 1024 i + 16 *
// lane.  The instruction offset applies to both addresses, so M0 is written
// once.  Inline assembly keeps the compiler from treating later LDS reads as
// dependent on the copies (it would wait for the next chunk's copies before
// reading the current slot); completion is waited for explicitly before the
// barrier of each chunk.  M0 is declared clobbered; one wait state separates
// the M0 write from the first copy.
__device__ __forceinline__ void copy_chunk(const char* base, const uint32_t (&voff)[4], uint32_t dst) {
  asm volatile(
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %4\n\t"
      "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
      "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
      "global_load_lds_dwordx4 %3, %4 offset:3072"
      :
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(base), "s"(dst)
      : "memory", "m0");
}

// The same copies with per-lane offsets that are not affine in i: one M0
// write per copy and no instruction offset, so every voff[i] is the full,
// non-negative byte offset of the lane's row piece from base.
__device__ __forceinline__ void copy_rows(const char* base, const uint32_t (&voff)[4], uint32_t dst) {
  asm volatile(
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %4\n\t"
      "s_add_u32 m0, %5, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %4\n\t"
      "s_add_u32 m0, %5, 0x800\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %4\n\t"
      "s_add_u32 m0, %5, 0xc00\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4"
      :
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(base), "s"(dst)
      : "memory", "scc", "m0");
}

// The 32 list entries of a gathered chunk (4 bytes per lane, lanes 0..31)
// into LDS at dst, as one more direct global->LDS copy: it completes with the
// chunk copies, before the barrier that ends the iteration.
__device__ __forceinline__ void copy_entries(const int32_t* base, uint32_t voff, uint32_t dst) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(dst)
      : "memory", "m0");
}

// This wave's copies have landed and its LDS reads have returned; after the
// barrier the same holds for the other wave, so both may read what was copied
// and rewrite what was read.
__device__ __forceinline__ void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One work item: query block u of head (b, h), both waves of the work-group.
// The next item's queue ticket is taken from *tkp by thread 0 at the start
// of this item's last chunk and left in *s_tk after its output stores.
template <int KIND>
__device__ __forceinline__ void attn_item(const AttnParams& P, const SampleView& S, const int h, const int u,
                                          lds_char* smem, int* tkp, int* s_tk) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int n = S.n;
  const int row0 = 64 * u;
  const int rw0 = row0 + 32 * wave;     // this wave's first row
  const int myrow = rw0 + l32;
  const int64_t hrow = S.q0 + (int64_t)h * n;     // this head's first row in Q, O and lse
  const size_t kvoff = (size_t)(S.kv0 + (int64_t)(h / P.gsz) * n) * kDH;
  const char* __restrict__ Kb = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(P.K) + kvoff);
  const char* __restrict__ Vb = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(P.V) + kvoff);

  // ---- Q^T operand in registers: lane l holds row myrow, 16-byte pieces 2t + hh
  u32x4 q[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(P.Q) +
                                                     (hrow + min(myrow, n - 1)) * (size_t)kDH);
    #pragma unroll
    for (int t = 0; t < 8; ++t) {
      q[t] = qp[2 * t + hh];
      if (myrow >= n) q[t] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- chunk lists of this item (wave-uniform)
  const ItemLists L = item_lists(P, S, h, KIND, u);
  const int Ca = __builtin_amdgcn_readfirstlane(L.Ca);
  const int Cb = __builtin_amdgcn_readfirstlane(L.Cb);
  const int Cf = __builtin_amdgcn_readfirstlane(L.Cf);
  const int C = Ca + Cb;
  if (C <= 0) {
    // nothing kept: o = 0, lse = -inf
    if (myrow < n) {
      const size_t obase = (hrow + myrow) * (size_t)kDH;
      #pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = 32 * c + 16 * hh;
        if (P.out_bf16) {
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(P.O) + obase + col / 2 * 2) = u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(P.O) + obase + col / 2 * 2 + 8) = u32x4{0, 0, 0, 0};
        } else {
          #pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(P.O) + obase + col + 4 * q4) = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (hh == 0 && P.lse) P.lse[hrow + myrow] = kNegInf;
    }
    if (threadIdx.x == 0) *s_tk = atomicAdd(tkp, 1);
    return;
  }
  const int sink_len = __builtin_amdgcn_readfirstlane(L.sink_len);
  const int wlo = __builtin_amdgcn_readfirstlane(L.wlo);
  const int whi = __builtin_amdgcn_readfirstlane(L.whi);
  const int win = __builtin_amdgcn_readfirstlane(L.win);
  const int ncols = __builtin_amdgcn_readfirstlane(L.ncols);
  const int rlast = rw0 + 31;     // this wave's last row
  const bool exact = KIND == MINF_VSLASH && P.slash_tile == 1;

  // Flags of a contiguous chunk whose keys kstart .. kstart+31 are kept
  // within [vlo, vhi], besides the causal limit and, for a window chunk
  // (w), the window limit of each row.  kNone may be conservative (unset
  // although nothing is kept); the per-element test is then exact.
  auto cflags = [&](int kstart, int vlo, int vhi, bool w) {
    // kFast iff 0 <= kstart <= n - 32 (both signs clear), kept in integer
    // arithmetic so that it stays on the scalar unit
    int f = ((kstart | (n - 32 - kstart)) >> 31) + 1;
    const int lo = w ? max(vlo, rw0 - win + 1) : vlo;
    if (lo > min(vhi, rlast)) return f | kNone;
    if (vlo > kstart || vhi < kstart + 31 || kstart + 31 > rw0 || (w && kstart < rlast - win + 1)) f |= kMask;
    return f;
  };
  // Chunk k of this item (wave-uniform), in two steps: fetch reads the list
  // entries it needs with scalar loads (a span's two offsets, a gathered
  // chunk's first and last column, a selected block), decode derives the
  // chunk from them.  In the steady loop the entries are fetched one
  // iteration before they are decoded, so the loads are never waited for.
  struct Raw { int a, b; };
  auto fetch = [&](int k) {
    Raw r{0, 0};
    if constexpr (KIND == MINF_VSLASH) {
      // span chunk: its two offsets; packed tail chunk: its first and last
      // offset; gathered columns: the first and last column
      if (k < Cf) {
        r.a = ld_uniform(L.clo, k);
        r.b = ld_uniform(L.chi, k);
      } else if (k < Ca) {
        const int e = 32 * (k - Cf);
        r.a = ld_uniform(L.tx, e);
        r.b = ld_uniform(L.tx, e + 31);
      } else {
        const int e = 32 * (k - Ca);
        const int cnt = min(32, ncols - e);
        r.a = ld_uniform(L.colrow, e);
        r.b = ld_uniform(L.colrow, e + cnt - 1);
      }
    } else if constexpr (KIND == MINF_BSPARSE) {
      r.a = ld_uniform(L.blkrow, k >> 1);
    }
    return r;
  };
  auto decode = [&](int k, const Raw& r) {
    Chunk d;
    if constexpr (KIND == MINF_ASHAPE) {
      const bool w = k >= Ca;
      d.kstart = w ? wlo + 32 * (k - Ca) : 32 * k;
      d.vlo = d.kstart;
      d.vhi = min(d.kstart + 31, w ? whi : sink_len - 1);
      d.flags = cflags(d.kstart, d.vlo, d.vhi, w) | (w ? kWin : 0);
    } else if constexpr (KIND == MINF_VSLASH) {
      if (k < Cf) {
        const int lo = r.a, hi = r.b;
        d.kstart = row0 - hi;
        d.vlo = max(0, d.kstart);
        d.vhi = min(row0 - lo, n - 1);
        d.flags = cflags(d.kstart, d.vlo, d.vhi, false);
        if (exact && !(d.flags & kNone)) d.flags |= kMask | kExact;
      } else if (k < Ca) {
        // packed tail chunk: keys 64u - x for its 32 ascending offsets x
        // (padding offsets give negative keys); the largest key comes from
        // the first offset, the smallest from the last
        const int kmax = row0 - r.a, kmin = row0 - r.b;
        d.kstart = k % 3;   // the LDS slot of its entries
        d.vlo = 0;
        d.vhi = 32;
        d.flags = kGather | kNeg | ((kmax < 0 || kmin > rlast) ? kNone : 0) | ((kmin < 0 || kmax > rw0) ? kMask : 0);
      } else {
        const int e = 32 * (k - Ca);
        const int cnt = min(32, ncols - e);
        const int gfirst = r.a, glast = r.b;
        d.kstart = k % 3;   // the LDS slot of its entries
        d.vlo = 0;
        d.vhi = cnt;
        d.flags = kGather | (gfirst > rlast ? kNone : 0) | ((cnt < 32 || glast > rw0) ? kMask : 0);
      }
    } else {
      const int vb = r.a;
      if (vb < 0 || vb > u) {   // not a causal block: keep nothing
        d.kstart = 0; d.vlo = 1; d.vhi = 0; d.flags = kNone;
      } else {
        d.kstart = 64 * vb + 32 * (k & 1);
        d.vlo = d.kstart;
        d.vhi = min(d.kstart + 31, n - 1);
        d.flags = cflags(d.kstart, d.vlo, d.vhi, false);
      }
    }
    return d;
  };
  // Plain chunks (32 keys inside [0, n), every pair of this wave's rows
  // kept: one affine copy, no per-element test) are recognised with a few
  // scalar comparisons; every other chunk takes the general decode above.
  // * A-shape window chunk at kstart: plain iff plo <= kstart <= phi, i.e.
  //   kstart >= rlast - w + 1 (inside every row's window), kstart + 31 <=
  //   rw0 (causal for the first row), kstart + 31 <= whi and <= n - 1.
  // * Block-Sparse: a selected block below the diagonal (0 <= vb < u).
  // * Vertical-Slash span chunk [lo, hi] of offsets: plain iff it is 32
  //   wide, kstart = 64u - hi >= 0, kstart + 31 <= min(rw0, n - 1), i.e.
  //   hi >= 31 - 32 * wave, and pairs are not tested one by one (exact).
  const int wbase = wlo - 32 * Ca;
  const int plo = max(rlast - win + 1, 0);
  const int phi = min(min(rw0, whi) - 31, n - 32);
  const int hmin = 31 - 32 * wave;
  auto decode_fast = [&](int k, const Raw& r) {
    if constexpr (KIND == MINF_ASHAPE) {
      const int ks = wbase + 32 * k;
      if (k >= Ca && ks >= plo && ks <= phi) return Chunk{ks, 0, 0, kFast};
    } else if constexpr (KIND == MINF_BSPARSE) {
      if (r.a >= 0 && r.a < u) return Chunk{64 * r.a + 32 * (k & 1), 0, 0, kFast};
    } else {
      const int ks = row0 - r.b;
      if (k < Cf && !exact && r.b - r.a == 31 && ks >= 0 && r.b >= hmin && ks <= n - 32)
        return Chunk{ks, 0, 0, kFast};
    }
    return decode(k, r);
  };
  auto describe = [&](int k) { return decode_fast(k, fetch(k)); };

  // ---- copy offsets.  Wave w copies rows 16w + 4i + lane/16 (i = 0..3) of
  //      each tile; lane l writes LDS piece l%16 of its row, which holds the
  //      row's piece (l%16) ^ swz(row).  The 1024 i of each copy is the
  //      instruction offset.
  const int crow0 = 16 * wave + (lane >> 4);
  const int cpiece = lane & 15;
  uint32_t koff[4], voff[4];
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = crow0 + 4 * i;
    koff[i] = (uint32_t)(r * kRowB + 16 * (cpiece ^ (r & 15)) - 1024 * i);
    voff[i] = (uint32_t)(r * kRowB + 16 * (cpiece ^ (4 * (r & 3))) - 1024 * i);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)smem + 4096 * wave;
  // the entry ring: gathered chunk k keeps its 32 list entries in slot k % 3
  // from two iterations before its K copy until the iteration of its V copy
  const uint32_t lst_base = (uint32_t)(uintptr_t)smem + kRing;
  auto copy_list = [&](int k) {
    if constexpr (KIND == MINF_VSLASH) {
      if (k >= Cf && wave == 0) {
        const int32_t* src = k < Ca ? L.tx + 32 * (k - Cf) : L.colrow + 32 * (k - Ca);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lst_base + kListB * (k % 3));
        if (lane < 32) copy_entries(src, 4 * lane, dst);
      }
    }
  };
  // K rows (V rows) of chunk d into the K (V) half of slot sl
  auto issue = [&](const Chunk& d, int sl, bool is_v) {
    const char* src = is_v ? Vb : Kb;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + sl * kSlotB + (is_v ? kTileB : 0));
    if (d.flags & kFast) {
      copy_chunk(src + (size_t)d.kstart * kRowB, is_v ? voff : koff, dst);
    } else {
      // per-lane rows: clamped into [0, n) (the excess keys are masked) or
      // gathered: the chunk's list entries were copied into the LDS entry
      // ring two iterations earlier (columns are keys, tail offsets x give
      // keys 64u - x).  (ks passes through an empty asm statement so that the
      // per-lane arithmetic is not hoisted above the branch onto the fast path)
      int ks = d.kstart;
      asm volatile("" : "+s"(ks));
      const lds_i32* ent = (const lds_i32*)(uintptr_t)(lst_base + kListB * ks);
      uint32_t o[4];
      #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = crow0 + 4 * i;
        int key = ks + r;
        if (d.flags & kNeg) key = row0 - ent[r];
        else if (d.flags & kGather) key = r < d.vhi ? ent[r] : 0;
        const uint32_t rb = (uint32_t)min(max(key, 0), n - 1) * kRowB;
        o[i] = rb + 16 * (cpiece ^ (is_v ? 4 * (r & 3) : (r & 15)));
      }
      copy_rows(src, o, dst);
    }
  };

  // Keep-bits of a chunk for this lane's row: bit 8a + b (a, b = 0..3) set
  // when the key at chunk position 8a + 4hh + b, which element 4a + b of
  // the lane holds, is kept.  Only for chunks with kMask; gathered chunks
  // read their list entries from the LDS entry ring.
  auto keep_bits = [&](const Chunk& d) -> uint32_t {
    if (!(d.flags & kMask) || (d.flags & kNone)) return 0u;
    if (d.flags & kGather) {
      // listed columns are keys; listed tail offsets x give keys 64u - x,
      // which may be negative (kept iff 0 <= key <= row)
      const bool neg = d.flags & kNeg;
      const lds_i32* ent = (const lds_i32*)(uintptr_t)(lst_base + kListB * d.kstart);
      uint32_t bits = 0;
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 8 * (i >> 2) + 4 * hh + (i & 3);
        const int e = pos < d.vhi ? ent[pos] : n;
        const int key = neg ? row0 - e : e;
        bits |= ((uint32_t)key <= (uint32_t)myrow ? 1u : 0u) << (8 * (i >> 2) + (i & 3));
      }
      return bits;
    }
    const int lo = ((d.flags & kWin) ? max(d.vlo, myrow - win + 1) : d.vlo) - d.kstart;
    const int hi = min(d.vhi, myrow) - d.kstart;
    const int a = max(lo, 0), z = min(hi, 31);
    uint32_t m = a > z ? 0u : ((0xffffffffu >> (31 - z)) & (0xffffffffu << a));
    if (d.flags & kExact) {
      // Eq. 5 taken literally: the pair (myrow, kstart + p) is kept iff
      // myrow - kstart - p is a selected offset or kstart + p a selected
      // column.  Offset bits: bit n + kBitsPad - 1 - myrow + kstart + p of
      // slash_bits, a 32-bit window of three words the wave reads together;
      // column bits: bit kstart + p + kBitsPad of col_bits.
      const uint32_t* sw = S.slash_bits + (int64_t)h * S.bits_words;
      const uint32_t* cw = S.col_bits + (int64_t)h * S.bits_words;
      const int w0 = (n + kBitsPad - 1 - rlast + d.kstart) >> 5;
      const uint32_t W0 = (uint32_t)ld_uniform((const int32_t*)sw, w0);
      const uint32_t W1 = (uint32_t)ld_uniform((const int32_t*)sw, w0 + 1);
      const uint32_t W2 = (uint32_t)ld_uniform((const int32_t*)sw, w0 + 2);
      const int sh = n + kBitsPad - 1 - myrow + d.kstart - 32 * w0;   // 0 .. 62
      const uint32_t dwin = sh < 32 ? __builtin_amdgcn_alignbit(W1, W0, sh) : __builtin_amdgcn_alignbit(W2, W1, sh - 32);
      const int cb = d.kstart + kBitsPad;
      const uint32_t C0 = (uint32_t)ld_uniform((const int32_t*)cw, cb >> 5);
      const uint32_t C1 = (uint32_t)ld_uniform((const int32_t*)cw, (cb >> 5) + 1);
      m &= dwin | __builtin_amdgcn_alignbit(C1, C0, cb & 31);
    }
    return m >> (4 * hh);
  };
  // exclusion (section 5.1): pairs outside the candidate set are -inf before
  // the maximum
  // A chunk without any kept pair for this wave (kNone) takes the same
  // in-place path with every keep-bit clear (keep_bits gives 0 for it), so
  // the scores are only ever rewritten where they stand.
  auto apply_mask = [&](floatx16& s, const Chunk& d, uint32_t bits) {
    if (d.flags & (kMask | kNone)) {
      // (the vector is reinterpreted whole: bit-casting single elements of a
      // vector has been miscompiled into reads of element 0)
      u32x16 v = __builtin_bit_cast(u32x16, s);
      #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 8 * (i >> 2) + (i & 3), 1);
        v[i] = (v[i] & keep) | (0xff800000u & ~keep);
      }
      s = __builtin_bit_cast(floatx16, v);
    }
  };
  // ---- operand read offsets within a slot
  // K: lane l reads row l%32, piece 2t + hh
  // V^T (transposing read): lane 16G + 4r + qq supplies row 16s + 8rho + 4(G/2) + r,
  // columns 32mb + 16(G%2) + 4qq .. +3 (the 16s + 8rho rows are instruction offsets)
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  uint32_t kofs[8], vofs[4];
  {
    const int G = lane >> 4, r = (lane >> 2) & 3, qq = lane & 3;
    #pragma unroll
    for (int t = 0; t < 8; ++t) kofs[t] = (uint32_t)(l32 * kRowB + 16 * ((2 * t + hh) ^ (l32 & 15)));
    #pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      vofs[mb] = (uint32_t)(kTileB + (4 * (G >> 1) + r) * kRowB + 16 * (4 * (mb ^ r) + 2 * (G & 1) + (qq >> 1)) +
                            8 * (qq & 1));
  }

  floatx16 acc[4];
  #pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    #pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m_run = kMInit, l_run = 0.f;
  const float cfac = P.c;
  // the rescale test compares raw scores against (m_run + tau) / c, so a
  // chunk needs no multiply or add for it (c > 0); the threshold changes only
  // with m_run
  const float inv_c = 1.0f / cfac;
  float thr = (m_run + kTau) * inv_c;

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto read_k = [&](int sl, u32x4 (&kop)[8]) {
    const uint32_t base = sbase + sl * kSlotB;
    #pragma unroll
    for (int t = 0; t < 8; ++t) kop[t] = *(lds_u32x4*)(uintptr_t)(base + kofs[t]);
  };
  auto read_v = [&](int sl, u32x4 (&vop)[2][4]) {
    #pragma unroll
    for (int st = 0; st < 2; ++st) {
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const lds_char* pv = (const lds_char*)(uintptr_t)(sbase + sl * kSlotB + vofs[mb]) + 4096 * st;
        const u32x2 lo = read_tr(pv);
        const u32x2 hi2 = read_tr(pv + 2048);
        vop[st][mb] = u32x4{lo[0], lo[1], hi2[0], hi2[1]};
      }
    }
  };
  auto qk = [&](const u32x4 (&kop)[8]) {
    floatx16 s;
    #pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    #pragma unroll
    for (int t = 0; t < 8; ++t) s = mma32(kop[t], q[t], s);
    return s;
  };

  // Walk order.  The 128 work-groups that run together on one XCD are
  // consecutive query blocks of one head and start together, so the order is
  // chosen to make them read nearby keys at nearby times (Eq. 7-8 do not
  // depend on the order):
  // * Vertical-Slash: chunks in list order, i.e. slash spans by descending
  //   key from the diagonal, then the gathered columns; block u's spans are
  //   block (u-1)'s shifted up by 64 keys (measured: 3.8% faster than the
  //   ascending walk at 128K, and equal at 1M);
  // * A-shape: block u's window is block (u+1)'s shifted down by two chunks,
  //   and a unit's blocks are queued from the last down, so block u starts
  //   2 (-u mod 128) chunks along: neighbours in a queue read the same keys
  //   at the same time, and the order depends on the block alone (a
  //   sequence gives the same bits wherever its items are queued);
  // * Block-Sparse: selected blocks from the last (the diagonal) down
  //   (3.4% faster than ascending at 512K).
  const int step = KIND == MINF_BSPARSE ? -1 : 1;
  int kc = KIND == MINF_ASHAPE ? (2 * (-u & 127)) % C : (KIND == MINF_BSPARSE ? C - 1 : 0);
  auto next_of = [&](int k) {
    k += step;
    return k == C ? 0 : (k < 0 ? C - 1 : k);
  };
  auto advance = [&]() { kc = next_of(kc); };

  // ---- software pipeline.  Chunk j lives in slot j%2 (K and V halves).  In
  //      iteration j the wave computes the softmax and P.V of chunk j and,
  //      interleaved with that softmax, the Q.K products of chunk j+1; the
  //      copies issued in iteration j are V of chunk j+1 and K of chunk j+2, so
  //      every slot half is rewritten only after both waves have passed the
  //      barrier that ends its last use.
  // list entries of the first three chunks (a gathered chunk among the
  // first two is read below, so those are waited for)
  copy_list(0);
  if (C > 1) copy_list(1);
  if (C > 2) copy_list(2);
  if (KIND == MINF_VSLASH && Cf < 2) wait_copies_and_barrier();
  Chunk d0 = describe(kc), d1{0, 1, 0, kNone}, d2{0, 1, 0, kNone};
  issue(d0, 0, false);
  issue(d0, 0, true);
  if (C > 1) {
    advance();
    d1 = describe(kc);
    issue(d1, 1, false);
  }
  // entries of the next chunk to decode (chunk 2), fetched ahead
  constexpr bool kPrefetch = KIND != MINF_ASHAPE;
  Raw rn{0, 0};
  if (kPrefetch && C > 2) rn = fetch(next_of(kc));
  wait_copies_and_barrier();
  uint32_t bits0 = keep_bits(d0);
  // the scores of chunk j live in sA for even j and in sB for odd j: each
  // iteration reads one and writes the other, so no copy between them
  floatx16 sA, sB;
  {
    u32x4 kop[8];
    read_k(0, kop);
    sA = qk(kop);
  }
  // iteration 0 rewrites the K half of slot 0, which both waves just read
  wait_copies_and_barrier();

  int tk = 0;   // thread 0: the next item's ticket
  // STEADY: chunks j+1 .. j+3 exist (j+1 .. j+2 for A-shape; no bound tests)
  auto iteration = [&](const int j, const int sl, auto steady, floatx16& s_cur, floatx16& s_nxt) {
    constexpr bool STEADY = decltype(steady)::value;
    // slot sl holds K and V of chunk j, slot sl^1 holds K of chunk j+1.
    // Kinds with list entries decode chunk j+2 from the entries fetched
    // during the previous iteration (already waited for before its barrier)
    // and fetch those of chunk j+3; A-shape chunks are pure arithmetic.
    u32x4 kop[8], vop[2][4];
    const bool more = STEADY || j + 1 < C;
    const bool more2 = STEADY || j + 2 < C;
    // the last chunk: take the next item's ticket now, so that its round trip
    // (and the item boundary) does not wait for this item's output stores
    if constexpr (!STEADY) {
      if (j == C - 1 && threadIdx.x == 0) tk = atomicAdd(tkp, 1);
    }
    read_k(sl ^ 1, kop);
    if constexpr (kPrefetch) {
      if (more2) {
        advance();
        d2 = decode_fast(kc, rn);
        if (STEADY || j + 3 < C) {
          rn = fetch(next_of(kc));
          copy_list(next_of(kc));
        }
      }
    }
    uint32_t bits1 = 0u;
    if (more) bits1 = keep_bits(d1);
    if (more) issue(d1, sl ^ 1, true);
    if constexpr (!kPrefetch) {
      if (more2) {
        advance();
        d2 = describe(kc);
      }
    }
    if (more2) issue(d2, sl, false);
    apply_mask(s_cur, d0, bits0);

    // online softmax of chunk j with lazy rescaling; the lane's maximum in
    // a tree of three-input maxima
    auto max3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
    const float mx = fmaxf(max3(max3(s_cur[0], s_cur[1], s_cur[2]), max3(s_cur[3], s_cur[4], s_cur[5]),
                                max3(s_cur[6], s_cur[7], s_cur[8])),
                           max3(max3(s_cur[9], s_cur[10], s_cur[11]), max3(s_cur[12], s_cur[13], s_cur[14]),
                                s_cur[15]));
    if (__builtin_amdgcn_ballot_w64(mx > thr)) {
      const float mxs = mx * cfac;
      const float pm = fmaxf(mxs, __shfl_xor(mxs, 32));      // the row's other 16 keys
      const float mn = pm > m_run + kTau ? pm : m_run;
      const float alpha = fast_exp2(m_run - mn);
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
      l_run *= alpha;
      m_run = mn;
      thr = (m_run + kTau) * inv_c;
    }
    // Q.K of chunk j+1 (8 products) interleaved with the exponentials,
    // conversions and row sums of chunk j (48 vector instructions)
    // (the wave holds a raised issue priority through its matrix products,
    // so that on a SIMD shared with another work-group's wave the products
    // of one keep the matrix unit busy while the other runs its scalar and
    // copy work: measured 4% faster at 128K)
    __builtin_amdgcn_s_setprio(1);
    s_nxt = qk(kop);
    read_v(sl, vop);
    u32x4 pb[2];
    #pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t w[4];
      #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0f = fast_exp2(__builtin_fmaf(s_cur[8 * st + 2 * e], cfac, -m_run));
        const float p1f = fast_exp2(__builtin_fmaf(s_cur[8 * st + 2 * e + 1], cfac, -m_run));
        w[e] = pack_bf16(p0f, p1f);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, l_run, false);
      }
      pb[st] = u32x4{w[0], w[1], w[2], w[3]};
    }
    // (the transposing V reads of chunk j go in after half of the products,
    // when half of the K operand registers are free)
    #pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);   // six vector instructions
      if (g == 3 || g == 7) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // eight LDS reads
    }
    // O^T += V^T P^T for chunk j
    #pragma unroll
    for (int st = 0; st < 2; ++st)
      #pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = mma32(vop[st][mb], pb[st], acc[mb]);
    __builtin_amdgcn_s_setprio(0);
    d0 = d1;
    d1 = d2;
    bits0 = bits1;
  };

  int j = 0;
  for (; j + (kPrefetch ? 4 : 3) < C; j += 2) {
    iteration(j, 0, std::true_type{}, sA, sB);
    wait_copies_and_barrier();
    iteration(j + 1, 1, std::true_type{}, sB, sA);
    wait_copies_and_barrier();
  }
  for (; j < C; j += 2) {
    iteration(j, 0, std::false_type{}, sA, sB);
    if (j + 1 >= C) break;
    wait_copies_and_barrier();
    iteration(j + 1, 1, std::false_type{}, sB, sA);
    if (j + 2 >= C) break;
    wait_copies_and_barrier();
  }

  // the next ticket, taken at the start of the last chunk, goes to LDS before
  // the output stores: waiting for it here waits for nothing else (the last
  // chunk issues no copies), whereas after the stores the wait would include
  // them (one counter covers loads and stores)
  if (threadIdx.x == 0) *s_tk = tk;

  // ---- finish: the row's sum over both lane halves, O = acc / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float f = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (myrow < n) {
    const size_t obase = (hrow + myrow) * (size_t)kDH;
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
      P.lse[hrow + myrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_d128_kernel(AttnParams P) {
  // persistent: take items from this XCD's queue until it is empty, then
  // from the other XCDs' queues in turn until all eight are
  int xq = blockIdx.x & 7;
  int hops = 0;
  int qoff = P.queue_meta[xq];
  int qcnt = P.queue_meta[8 + xq];
  __shared__ __attribute__((aligned(16))) char smem_g[kSmem];
  lds_char* smem = (lds_char*)smem_g;
  // tickets: the first here, each next one by the item before it (during its
  // last chunk), published in LDS after that item's output stores.  The
  // barriers between items wait for LDS only: the output stores complete
  // while the next item loads its lists.
  int* s_tk = reinterpret_cast<int*>(smem_g + kTicket);
  int* tkp = &P.queue_meta[16 + xq];
  if (threadIdx.x == 0) *s_tk = atomicAdd(tkp, 1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  while (true) {
    const int qi = __builtin_amdgcn_readfirstlane(*s_tk);
    // both waves hold qi before the ticket word is written again
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (qi >= qcnt) {
      // this queue is drained: the work-group helps with the next XCD's
      // queue (its items run from keys cached in another L2, but only while
      // the queues run out, when the XCDs would otherwise finish unevenly)
      if (++hops == 8) break;
      xq = __builtin_amdgcn_readfirstlane((xq + 1) & 7);
      qoff = __builtin_amdgcn_readfirstlane(P.queue_meta[xq]);
      qcnt = __builtin_amdgcn_readfirstlane(P.queue_meta[8 + xq]);
      tkp = &P.queue_meta[16 + xq];
      if (threadIdx.x == 0) *s_tk = atomicAdd(tkp, 1);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      continue;
    }
    const int item = ld_uniform(P.queue, (int64_t)qoff + qi);
    const int bhi = item / P.nq;
    const int u = item % P.nq;
    const int b = bhi / P.Hq;
    const int h = bhi % P.Hq;
    const int kind = __builtin_amdgcn_readfirstlane(P.ht.kind[h]);
    const SampleView S = sample_view(P, b);
    if (kind == MINF_VSLASH) attn_item<MINF_VSLASH>(P, S, h, u, smem, tkp, s_tk);
    else if (kind == MINF_BSPARSE) attn_item<MINF_BSPARSE>(P, S, h, u, smem, tkp, s_tk);
    else attn_item<MINF_ASHAPE>(P, S, h, u, smem, tkp, s_tk);
    // the next item reuses the LDS rings and reads the ticket
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

hipError_t launch_attn_bf16_d128(const AttnParams& p, hipStream_t st) {
  static int wgs = 0;
  if (!wgs) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    wgs = ((4 * cus + 7) / 8) * 8;   // four two-wave work-groups per CU
  }
  hipLaunchKernelGGL(attn_cost_kernel, dim3(p.sched_units), dim3(256), 0, st, p);
  hipLaunchKernelGGL(attn_sched_kernel, dim3(1), dim3(256), 0, st, p);
  hipLaunchKernelGGL(attn_fill_kernel, dim3(p.sched_units), dim3(256), 0, st, p);
  timing_mark(st, 0);
  hipLaunchKernelGGL(attn_bf16_d128_kernel, dim3(wgs), dim3(128), 0, st, p);
  timing_mark(st, 1);
  return hipGetLastError();
}

}  // namespace minf
