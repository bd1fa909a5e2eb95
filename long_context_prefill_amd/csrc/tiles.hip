// Index -> tile lists, and exact kept-edge counts.
//
// PaperTrace 2.1.2 "MInference", section 4.1 and blog-zz7 "LLM模型之MInference"
// section 2.3.3 ("get Vertical-Slash index"): the selected slash offsets are
// covered by square tiles (ranges), the verticals are points; ranges are
// merged and a vertical that already lies inside a selected range is dropped
// from the column list so that no (query, key) pair enters the softmax twice.
//
// Slash expansion used here: offset d covers, for query block u (64 rows), the
// keys [64u - d, 64u + 63 - d].  Key j of block u is therefore covered iff
// x = 64u - j lies in S = union over d of [d - 63, d].  S does not depend on
// u, so the merged ranges of S are built once per head and every query block
// reads them shifted by 64u.  The ranges are also cut into chunks of at most
// 32 offsets (the attention kernel's unit of work); block u uses the chunks
// whose lowest offset is <= 64u.
//
// Kept edges E_h = sum_i |N_h(i)| (section 1.2 of the page) are counted in
// closed form per query block: slash keys through prefix counts of S, plus
// the uncovered verticals, plus the block areas of Block-Sparse heads, plus
// the A-shape formula sum_i min(i+1, g+w) (Eq. 4).  Under exact slash pairs
// (slash_tile == 1, Eq. 5 taken literally) the tile lists stay the same (the
// pairs of offset d in block u lie inside [64u - d, 64u + 63 - d]); the
// attention then tests each pair against per-head offset and column
// bitmaps, and E_h is counted from the two sorted lists.
#include "kernels.h"

namespace minf {


__device__ __forceinline__ int64_t ashape_edges(int64_t n, int64_t g, int64_t w) {
  const int64_t m = g + w;       // |N(i)| = min(i+1, g+w)
  if (n <= m) return n * (n + 1) / 2;
  return m * (m + 1) / 2 + (n - m) * m;
}

// Block-wide exclusive scan of one int per thread (256 threads), returns the
// total through *total: an inclusive scan inside each wave by shuffles, then
// the four wave totals through LDS (two barriers; sh holds 4 ints).
__device__ int block_exscan(int x, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int v = x;
  #pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0, tot = 0;
  #pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = sh[i];
    before += i < w ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();     // sh is reused by the next call
  return before + v - x;
}

// The list kernels below take kIPT consecutive entries per thread and round
// (256 kIPT entries per round), with every load of a round issued before its
// first use, so a round costs one memory latency rather than kIPT.
constexpr int kIPT = 8;
constexpr int kRound = 256 * kIPT;

// Last index r in [0, cnt) with a[r * step] <= x (ascending), -1 if none,
// found by one wave: up to 64 sampled entries per round, so a list of up to
// 4096 entries costs two rounds of loads instead of a dependent chain of
// twelve.
__device__ __forceinline__ int wave_last_le(const int32_t* a, int cnt, int x, int step = 1) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = cnt;   // the answer lies in [lo - 1, hi - 1]; a[lo - 1] <= x when lo > 0
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) / 64;
    const int k = lo + lane * stride;
    const int c = __popcll(__ballot(k < hi && a[(int64_t)k * step] <= x));   // entries <= x form a prefix
    if (c == 0) { hi = lo; break; }
    const int nlo = lo + (c - 1) * stride;
    hi = min(hi, nlo + stride);
    lo = nlo;
  }
  const int k = lo + lane;
  return lo - 1 + __popcll(__ballot(k < hi && a[(int64_t)k * step] <= x));
}

// 1) validate indices, initialise kept_edges, merge slash ranges.
__global__ __launch_bounds__(256) void vs_ranges_kernel(TileParams P) {
  __shared__ int sh[256];
  __shared__ int bad_s, bad_v;
  const int bh = blockIdx.x;
  const int h = bh % P.Hq;
  const int kind = P.ht.kind[h];
  if (threadIdx.x == 0) {
    int64_t e = 0;
    if (kind == MINF_ASHAPE) e = ashape_edges(P.n, P.ht.a[h], P.ht.b[h]);
    P.t.kept_edges[bh] = e;
    bad_s = 0; bad_v = 0;
  }
  if (kind != MINF_VSLASH) return;
  const int nv = P.ht.b[h], ns = P.ht.c[h];
  const int32_t* offs = P.slash_idx + (size_t)bh * P.max_s;
  const int32_t* cols = P.vert_idx + (size_t)bh * P.max_v;
  __syncthreads();
  // each list must lie in [0, n) and ascend strictly
  auto check = [&](const int32_t* a, int cnt, int* bad) {
    for (int base = 0; base < cnt; base += kRound) {
      const int k0 = base + (int)threadIdx.x * kIPT;
      int v[kIPT + 1];   // entries k0 - 1 .. k0 + kIPT - 1
      #pragma unroll
      for (int e = 0; e <= kIPT; ++e) {
        const int k = k0 - 1 + e;
        v[e] = (k >= 0 && k < cnt) ? a[k] : 0;
      }
      #pragma unroll
      for (int e = 1; e <= kIPT; ++e) {
        const int k = k0 - 1 + e;
        if (k < cnt && (v[e] < 0 || v[e] >= P.n || (k > 0 && v[e - 1] >= v[e]))) *bad = 1;
      }
    }
  };
  check(offs, ns, &bad_s);
  check(cols, nv, &bad_v);
  __syncthreads();
  const bool ok = !(bad_s || bad_v);
  if (threadIdx.x == 0) {
    P.head_ok[bh] = ok ? 1 : 0;
    if (!ok) atomicOr(P.t.status, (bad_s ? MINF_DEV_BAD_SLASH : 0) | (bad_v ? MINF_DEV_BAD_VERTICAL : 0));
  }
  int carry = 0;   // ranges emitted so far
  if (ok) {
    // offset k starts a range when k = 0 or it lies more than 64 above the
    // previous one, and ends one when k = ns - 1 or the next lies more than
    // 64 above it
    int32_t* slo = P.t.span_lo + (size_t)bh * P.max_s;
    int32_t* shi = P.t.span_hi + (size_t)bh * P.max_s;
    for (int base = 0; base < ns; base += kRound) {
      const int k0 = base + (int)threadIdx.x * kIPT;
      int v[kIPT + 2];   // entries k0 - 1 .. k0 + kIPT
      #pragma unroll
      for (int e = 0; e < kIPT + 2; ++e) {
        const int k = k0 - 1 + e;
        v[e] = (k >= 0 && k < ns) ? offs[k] : 0;
      }
      int starts = 0;
      #pragma unroll
      for (int e = 1; e <= kIPT; ++e) {
        const int k = k0 - 1 + e;
        starts += (k < ns) && (k == 0 || v[e] - v[e - 1] > 64);
      }
      int tot;
      int pos = carry + block_exscan(starts, sh, &tot);   // ranges started before this thread's entries
      #pragma unroll
      for (int e = 1; e <= kIPT; ++e) {
        const int k = k0 - 1 + e;
        if (k < ns) {
          const int flag = (k == 0) || (v[e] - v[e - 1] > 64);
          if (flag) slo[pos] = v[e] - 63;
          const bool last = (k == ns - 1) || (v[e + 1] - v[e] > 64);
          if (last) shi[pos + flag - 1] = v[e];
          pos += flag;
        }
      }
      carry += tot;
    }
  }
  if (threadIdx.x == 0) P.t.span_cnt[bh] = ok ? carry : 0;
}

// Last index r in [0, cnt) with a[r] <= x (a ascending), -1 if none: one
// thread's binary search.
__device__ __forceinline__ int last_le(const int32_t* a, int cnt, int x) {
  int l = 0, r = cnt;
  while (l < r) { const int m = (l + r) >> 1; if (a[m] <= x) l = m + 1; else r = m; }
  return l - 1;
}

constexpr int kSlabWords = 8192;   // bitmap words built in LDS at a time (32 per thread)

// Bits [s, e] (0 <= s <= e <= 31) of a 32-bit word.
__device__ __forceinline__ uint32_t bit_span(int s, int e) {
  return (e - s + 1 == 32) ? 0xffffffffu : (((1u << (e - s + 1)) - 1u) << s);
}

// 2) cut ranges into chunks, prefix counts, coverage bitmap.  Each range is
//    cut into whole 32-offset chunks from its low end; the shorter last
//    piece (its tail) goes to the per-head tail list, whose entries the
//    attention packs 32 to a chunk (under exact slash pairs the tail stays a
//    chunk of its own: the per-pair test needs contiguous keys).  The
//    chunks, the tail entries and the bitmap words are written by all
//    threads evenly: each takes a contiguous share
//    of them, finds its first range once and walks on, so a long range does
//    not fall to one thread.
__global__ __launch_bounds__(256) void vs_chunks_kernel(TileParams P) {
  __shared__ int sh[256];
  const int bh = blockIdx.x;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const bool tails = P.slash_tile != 1;
  const int nr = P.t.span_cnt[bh];
  const int32_t* lo = P.t.span_lo + (size_t)bh * P.max_s;
  const int32_t* hi = P.t.span_hi + (size_t)bh * P.max_s;
  int32_t* cum = P.span_cum + (size_t)bh * (P.max_s + 1);
  int32_t* rch = P.range_chunks + (size_t)bh * (P.max_s + 1);
  int32_t* rtl = P.range_tails + (size_t)bh * (P.max_s + 1);
  int32_t* clo = P.t.chunk_lo + (size_t)bh * P.max_chunks;
  int32_t* chi = P.t.chunk_hi + (size_t)bh * P.max_chunks;
  int32_t* tx = P.t.tail_x + (size_t)bh * P.max_tail;
  auto nchunks = [&](int a, int b) { const int w = b - a + 1; return tails ? (w >> 5) : ((w + 31) >> 5); };
  auto ntail = [&](int a, int b) { return tails ? ((b - a + 1) & 31) : 0; };
  auto ncov = [&](int a, int b) { return b >= 0 ? b - max(a, 0) + 1 : 0; };
  // prefix counts of chunks, covered offsets >= 0 and tail entries per range
  int carry_c = 0, carry_x = 0, carry_t = 0;
  for (int base = 0; base < nr; base += kRound) {
    const int r0 = base + (int)threadIdx.x * kIPT;
    int a[kIPT], b[kIPT];
    #pragma unroll
    for (int e = 0; e < kIPT; ++e) {
      const int r = r0 + e;
      a[e] = r < nr ? lo[r] : 0;
      b[e] = r < nr ? hi[r] : -1;
    }
    int sc = 0, sx = 0, st = 0;
    #pragma unroll
    for (int e = 0; e < kIPT; ++e) {
      if (r0 + e < nr) { sc += nchunks(a[e], b[e]); sx += ncov(a[e], b[e]); st += ntail(a[e], b[e]); }
    }
    int tc, tx_, tt;
    int pc = carry_c + block_exscan(sc, sh, &tc);
    int px = carry_x + block_exscan(sx, sh, &tx_);
    int pt = carry_t + block_exscan(st, sh, &tt);
    #pragma unroll
    for (int e = 0; e < kIPT; ++e) {
      const int r = r0 + e;
      if (r < nr) {
        rch[r] = pc;
        cum[r] = px;
        rtl[r] = pt;
        pc += nchunks(a[e], b[e]);
        px += ncov(a[e], b[e]);
        pt += ntail(a[e], b[e]);
      }
    }
    carry_c += tc;
    carry_x += tx_;
    carry_t += tt;
  }
  if (threadIdx.x == 0) {
    rch[nr] = carry_c; cum[nr] = carry_x; rtl[nr] = carry_t;
    if (carry_c > P.max_chunks) atomicOr(P.t.status, MINF_DEV_CAPACITY);
  }
  __syncthreads();   // the prefix arrays are read by every thread below
  const int nthr = (int)blockDim.x, tid = (int)threadIdx.x;
  // chunks: chunk c of range r (rch[r] <= c < rch[r+1]) holds offsets
  // lo[r] + 32 (c - rch[r]) .. +31, clipped to the range
  {
    const int tot = (int)min<long long>(carry_c, P.max_chunks);
    const int per = (tot + nthr - 1) / nthr, c0 = tid * per, c1 = min(tot, c0 + per);
    if (c0 < c1) {
      int r = last_le(rch, nr, c0);
      int next = rch[r + 1], a = lo[r], b = hi[r], first = rch[r];
      for (int c = c0; c < c1; ++c) {
        while (c >= next) { ++r; first = next; next = rch[r + 1]; a = lo[r]; b = hi[r]; }
        const int m = c - first;
        clo[c] = a + 32 * m;
        chi[c] = min(a + 32 * m + 31, b);
      }
    }
  }
  // tail entries: entry i of range r (rtl[r] <= i < rtl[r+1]) is the offset
  // after the range's whole chunks; then the padding to whole packed chunks
  const int tpad = (carry_t + 31) & ~31;
  {
    const int per = (tpad + nthr - 1) / nthr, i0 = tid * per, i1 = min(tpad, i0 + per);
    if (i0 < i1) {
      int r = carry_t > 0 ? last_le(rtl, nr, min(i0, carry_t - 1)) : 0;
      int next = nr > 0 ? rtl[r + 1] : 0, first = nr > 0 ? rtl[r] : 0;
      int xs = nr > 0 ? lo[r] + 32 * nchunks(lo[r], hi[r]) : 0;
      for (int i = i0; i < i1; ++i) {
        int v = MINF_TAIL_PAD;
        if (i < carry_t) {
          while (i >= next) { ++r; first = next; next = rtl[r + 1]; xs = lo[r] + 32 * nchunks(lo[r], hi[r]); }
          v = xs + (i - first);
        }
        if (i < P.max_tail) tx[i] = v;
      }
    }
  }
  if (threadIdx.x == 0) {
    P.t.tail_cnt[bh] = (int)min<long long>(carry_t, P.max_tail);
    if (tpad > P.max_tail) atomicOr(P.t.status, MINF_DEV_CAPACITY);
  }
  // coverage bitmap over x in [-63, n): bit x + 63.  Word w holds bits
  // 32w .. 32w + 31; the ranges meeting it are the first range ending at or
  // after its first bit and, ranges being at least 64 bits wide, at most the
  // one after it.  Slabs of kSlabWords words: each thread builds 32
  // consecutive words in LDS, walking the ranges with the current and the
  // next one in registers, and the slab is written out whole.
  uint32_t* bm = P.bitmap + (size_t)bh * P.bm_words;
  __shared__ uint32_t slab[kSlabWords];
  constexpr int kBig = 1 << 29;      // beyond every range
  for (int64_t s0 = 0; s0 < P.bm_words; s0 += kSlabWords) {
    const int nw = (int)min<int64_t>(kSlabWords, P.bm_words - s0);
    const int w0 = 32 * tid;
    if (w0 < nw) {
      const int b00 = 32 * (int)(s0 + w0);
      // first range r with hi[r] + 63 >= b00
      int l = 0, rr = nr;
      while (l < rr) { const int m = (l + rr) >> 1; if (hi[m] + 63 < b00) l = m + 1; else rr = m; }
      int r = l;
      int la = r < nr ? lo[r] + 63 : kBig, ha = r < nr ? hi[r] + 63 : kBig;
      int lb = r + 1 < nr ? lo[r + 1] + 63 : kBig, hb = r + 1 < nr ? hi[r + 1] + 63 : kBig;
      for (int w = w0; w < min(nw, w0 + 32); ++w) {
        const int b0 = 32 * (int)(s0 + w), b1 = b0 + 31;
        while (ha < b0) {
          ++r;
          la = lb; ha = hb;
          lb = r + 1 < nr ? lo[r + 1] + 63 : kBig;
          hb = r + 1 < nr ? hi[r + 1] + 63 : kBig;
        }
        uint32_t bits = 0;
        if (la <= b1) bits |= bit_span(max(la, b0) - b0, min(ha, b1) - b0);
        if (lb <= b1) bits |= bit_span(max(lb, b0) - b0, min(hb, b1) - b0);
        slab[w] = bits;
      }
    }
    __syncthreads();
    for (int w = tid; w < nw; w += nthr) bm[s0 + w] = slab[w];
    __syncthreads();   // the slab is rebuilt for the next words
  }
}

__device__ __forceinline__ bool covered(const uint32_t* bm, int x) {
  const int i = x + 63;
  return (bm[i >> 5] >> (i & 31)) & 1u;
}

// 3) per query block: chunk count, uncovered verticals, kept edges (VS).
//    One wave per query block; the columns are read four rounds of 64 at a
//    time, each round's loads (column, then coverage word) issued together.
__global__ __launch_bounds__(256) void vs_cols_kernel(TileParams P) {
  const int bh = blockIdx.y;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + wave;
  __shared__ unsigned long long part[4];
  unsigned long long edges = 0;
  if (u < P.nq) {
    const int row0 = 64 * u;
    const int Lu = min(64, P.n - row0);
    const int row_end = row0 + Lu - 1;
    const size_t bu = (size_t)bh * P.nq + u;
    const bool ok = P.head_ok[bh] != 0;
    const int nr = ok ? P.t.span_cnt[bh] : 0;
    const int32_t* lo = P.t.span_lo + (size_t)bh * P.max_s;
    const int32_t* hi = P.t.span_hi + (size_t)bh * P.max_s;
    const int32_t* cum = P.span_cum + (size_t)bh * (P.max_s + 1);
    const int32_t* rch = P.range_chunks + (size_t)bh * (P.max_s + 1);
    const uint32_t* bm = P.bitmap + (size_t)bh * P.bm_words;
    // last range with lo <= 64u
    const int X = row0;
    const int rs = wave_last_le(lo, nr, X);   // -1 if none
    int ccnt = 0;
    long long cov_pos = 0;  // |S intersect [0, X]|
    if (rs >= 0) {
      const int l = lo[rs], hh = hi[rs], rc = rch[rs], cu = cum[rs];
      const int w = hh - l + 1;
      const bool tails = P.slash_tile != 1;
      ccnt = rc + min(tails ? (w >> 5) : ((w + 31) >> 5), ((X - l) >> 5) + 1);
      const int e = min(hh, X), s = max(l, 0);
      cov_pos = cu + (e >= s ? e - s + 1 : 0);
    }
    ccnt = min<long long>(ccnt, P.max_chunks);
    // packed tail chunks whose first entry is <= 64u
    const int32_t* tx = P.t.tail_x + (size_t)bh * P.max_tail;
    const int npk = ok ? (int)min<long long>((P.t.tail_cnt[bh] + 31) >> 5, P.max_tail >> 5) : 0;
    const int pk = wave_last_le(tx, npk, X, 32) + 1;
    // span edges: Lu per covered x >= 0 with x <= 64u, and max(0, Lu + x)
    // for x in [-63, -1] (lane l takes x = l - 63)
    if (lane == 0) {
      edges += (long long)Lu * cov_pos;
      P.t.chunk_cnt[bu] = ccnt;
      P.t.pk_cnt[bu] = pk;
    }
    if (nr > 0 && lane < 63) {
      const int x = lane - 63;
      if (Lu + x > 0 && covered(bm, x)) edges += Lu + x;
    }
    // uncovered verticals of this block, ascending
    const int nv = ok ? P.ht.b[h] : 0;
    const int32_t* cols = P.vert_idx + (size_t)bh * P.max_v;
    int32_t* out = P.t.cols + bu * P.max_v;
    int cnt = 0;
    bool done = false;
    for (int base = 0; base < nv && !done; base += 256) {
      int c[4];
      uint32_t wd[4];
      #pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = base + 64 * j + lane;
        c[j] = k < nv ? cols[k] : 0x7fffffff;
      }
      #pragma unroll
      for (int j = 0; j < 4; ++j) {
        // x = row0 - c lies in [-63, n) for an in-range column
        const int i = row0 - c[j] + 63;
        wd[j] = c[j] <= row_end ? bm[i >> 5] : 0xffffffffu;
      }
      #pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (done) break;
        const bool in_range = c[j] <= row_end;
        const int i = row0 - c[j] + 63;
        const bool keep = in_range && !((wd[j] >> (i & 31)) & 1u);
        const unsigned long long m = __ballot(keep);
        const int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
        if (keep) {
          out[pos] = c[j];
          edges += row_end - max(c[j], row0) + 1;
        }
        cnt += __popcll(m);
        if (__any(!in_range)) done = true;   // columns are ascending: the rest lie beyond the block
      }
    }
    if (lane == 0) P.t.col_cnt[bu] = cnt;
    if (P.slash_tile == 1) edges = 0;   // exact slash pairs: counted by vs_exact_edges_kernel
  }
  // reduce edges over the work-group, one atomic per group (integer: order-free)
  for (int off = 32; off > 0; off >>= 1) edges += __shfl_xor(edges, off);
  if (lane == 0) part[wave] = edges;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long tot = part[0] + part[1] + part[2] + part[3];
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(P.t.kept_edges + bh), tot);
  }
}

// 3b) exact slash pairs (slash_tile == 1, Eq. 5): the per-head bitmaps the
//     attention tests each span pair against.  Bit n + kBitsPad - 1 - d of
//     slash_bits marks offset d, bit j + kBitsPad of col_bits column j.
//     One thread per 32-bit word, both lists ascending.
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int cnt, int x) {
  int l = 0, r = cnt;
  while (l < r) { const int m = (l + r) >> 1; if (a[m] < x) l = m + 1; else r = m; }
  return l;
}

__global__ __launch_bounds__(256) void vs_bits_kernel(TileParams P) {
  const int bh = blockIdx.y;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH) return;
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= P.bits_words) return;
  const bool ok = P.head_ok[bh] != 0;
  uint32_t sb = 0, cb = 0;
  if (ok) {
    const int n = P.n;
    const int b0 = (int)(32 * w);
    // offsets d with bit n + kBitsPad - 1 - d in [b0, b0 + 31]
    const int ns = P.ht.c[h];
    const int32_t* offs = P.slash_idx + (size_t)bh * P.max_s;
    const int dlo = n + kBitsPad - 1 - (b0 + 31), dhi = n + kBitsPad - 1 - b0;
    for (int k = lower_bound_i32(offs, ns, dlo); k < ns && offs[k] <= dhi; ++k)
      sb |= 1u << (n + kBitsPad - 1 - offs[k] - b0);
    // columns j with bit j + kBitsPad in [b0, b0 + 31]
    const int nv = P.ht.b[h];
    const int32_t* cols = P.vert_idx + (size_t)bh * P.max_v;
    const int jlo = b0 - kBitsPad, jhi = b0 - kBitsPad + 31;
    for (int k = lower_bound_i32(cols, nv, jlo); k < nv && cols[k] <= jhi; ++k)
      cb |= 1u << (cols[k] + kBitsPad - b0);
  }
  P.t.slash_bits[(size_t)bh * P.bits_words + w] = sb;
  P.t.col_bits[(size_t)bh * P.bits_words + w] = cb;
}

// 3c) kept edges under exact slash pairs: sum_i |{j <= i : i - j in D} u
//     {j <= i : j in C}| = sum_d (n - d) + sum_c (n - c) - #{(c, d) : c + d <= n-1}.
__global__ __launch_bounds__(256) void vs_exact_edges_kernel(TileParams P) {
  const int bh = blockIdx.x;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_VSLASH || !P.head_ok[bh]) return;
  const int n = P.n;
  const int ns = P.ht.c[h], nv = P.ht.b[h];
  const int32_t* offs = P.slash_idx + (size_t)bh * P.max_s;
  const int32_t* cols = P.vert_idx + (size_t)bh * P.max_v;
  long long e = 0;
  for (int k = threadIdx.x; k < ns; k += 256) e += n - offs[k];
  for (int k = threadIdx.x; k < nv; k += 256) {
    const int c = cols[k];
    // offsets d <= n - 1 - c: pairs (c, d) whose key c is also at offset d of row c + d
    const int both = lower_bound_i32(offs, ns, n - c);
    e += (long long)(n - c) - both;
  }
  __shared__ long long part[4];
  for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = e;
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long tot = part[0] + part[1] + part[2] + part[3];
    atomicAdd(reinterpret_cast<unsigned long long*>(P.t.kept_edges + bh), (unsigned long long)tot);
  }
}

// 4) Block-Sparse: validate J_u and count the kept block areas.
__global__ __launch_bounds__(256) void bs_edges_kernel(TileParams P) {
  const int bh = blockIdx.y;
  const int h = bh % P.Hq;
  if (P.ht.kind[h] != MINF_BSPARSE) return;
  const int u = blockIdx.x * 256 + threadIdx.x;
  __shared__ unsigned long long part[4];
  unsigned long long edges = 0;
  if (u < P.nq) {
    const size_t bu = (size_t)bh * P.nq + u;
    const int cnt = P.blk_cnt[bu];
    const int Lu = min(64, P.n - 64 * u);
    bool bad = cnt < 0 || cnt > P.max_kb || cnt > u + 1;
    const int32_t* J = P.blk_idx + bu * P.max_kb;
    int prev = -1;
    for (int i = 0; !bad && i < cnt; ++i) {
      const int v = J[i];
      if (v <= prev || v > u) { bad = true; break; }
      edges += (v < u) ? (unsigned long long)Lu * 64ull : (unsigned long long)(Lu * (Lu + 1) / 2);
      prev = v;
    }
    if (bad) { atomicOr(P.t.status, MINF_DEV_BAD_BLOCK); edges = 0; }
  }
  for (int off = 32; off > 0; off >>= 1) edges += __shfl_xor(edges, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = edges;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long tot = part[0] + part[1] + part[2] + part[3];
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(P.t.kept_edges + bh), tot);
  }
}

hipError_t launch_tiles(const TileParams& p, bool has_vs, bool has_bs, hipStream_t st) {
  const unsigned BH = (unsigned)(p.B * p.Hq);
  hipLaunchKernelGGL(vs_ranges_kernel, dim3(BH), dim3(256), 0, st, p);
  if (has_vs) {
    hipLaunchKernelGGL(vs_chunks_kernel, dim3(BH), dim3(256), 0, st, p);
    hipLaunchKernelGGL(vs_cols_kernel, dim3((p.nq + 3) / 4, BH), dim3(256), 0, st, p);
    if (p.slash_tile == 1) {
      hipLaunchKernelGGL(vs_bits_kernel, dim3((unsigned)((p.bits_words + 255) / 256), BH), dim3(256), 0, st, p);
      hipLaunchKernelGGL(vs_exact_edges_kernel, dim3(BH), dim3(256), 0, st, p);
    }
  }
  if (has_bs) hipLaunchKernelGGL(bs_edges_kernel, dim3((p.nq + 255) / 256, BH), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace minf
