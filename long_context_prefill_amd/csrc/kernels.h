// Kernel parameter blocks and launchers shared between the host entry points
// and the kernel translation units.
#pragma once

#include "common.h"

namespace minf {

// Left padding, in bits, of the exact-slash bitmaps (minf_tiles.slash_bits,
// col_bits): offset d sits at bit n + kBitsPad - 1 - d, column j at bit
// j + kBitsPad, so every 32-bit window a chunk needs starts at bit >= 0.
constexpr int kBitsPad = 128;
inline int64_t exact_bits_words(int n) { return ((int64_t)n + 2 * kBitsPad + 64 + 31) / 32 + 2; }

// ---------------------------------------------------------------- attention
// One sequence of a ragged batch, as the attention kernels see it: its
// length, where its rows start in the packed Q, K, V, O and lse tensors, and
// its own index and tile lists (each laid out as for a B = 1 problem of
// length n, with that problem's capacities).
struct SampleDesc {
  int64_t q_row;        // first row of the sample's [Hq, n] rows of Q, O and lse (rows of dh elements in Q, O)
  int64_t kv_row;       // first row of its [Hkv, n] rows of K and V
  const int32_t* chunk_lo;
  const int32_t* chunk_hi;
  const int32_t* chunk_cnt;
  const int32_t* cols;
  const int32_t* col_cnt;
  const int32_t* blk_idx;
  const int32_t* blk_cnt;
  const uint32_t* slash_bits;
  const uint32_t* col_bits;
  const int32_t* tail_x;
  const int32_t* pk_cnt;
  int64_t max_chunks, max_v, max_kb, bits_words, max_tail;
  int32_t n, nq;
};
constexpr int kSampleBatch = 16;     // descriptors written per launch of the table writer
struct SampleBatch {
  SampleDesc d[kSampleBatch];
  SampleDesc* dst;
  int32_t count;
};
// dst[0 .. count) = d[0 .. count) (attn.hip), a plain kernel, so that the
// table needs no host-to-device copy.
hipError_t launch_write_samples(const SampleBatch& b, hipStream_t st);

struct AttnParams {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  const int32_t* blk_idx;
  const int32_t* blk_cnt;
  const int32_t* chunk_lo;
  const int32_t* chunk_hi;
  const int32_t* chunk_cnt;
  const int32_t* cols;
  const int32_t* col_cnt;
  const int32_t* tail_x;     // [B,Hq,max_tail] packed tail offsets (minf_tiles.tail_x)
  const int32_t* pk_cnt;     // [B,Hq,nq] packed chunks per block
  int64_t max_kb, max_chunks, max_v, max_tail;
  int32_t B, Hq, Hkv, n, nq, gsz;
  int32_t n_utiles, n_segs;
  float c;          // scale * log2(e)
  int32_t out_bf16;
  HeadTable ht;     // ASHAPE: a = sink, b = window
  // per-XCD work queues (attn_bf16.hip); units are (b*Hq + h) * sched_P + part,
  // part covering query blocks [part*sched_R, (part+1)*sched_R)
  int64_t* sched_cost;      // ws [sched_units]
  int32_t* sched_order;     // ws [sched_units]
  int32_t* unit_xcd;        // ws [sched_units], -1 = no items
  int32_t* unit_off;        // ws [sched_units]: first item within its XCD's queue
  int32_t* queue;           // ws [B*Hq*nq]: items b*Hq*nq + h*nq + u
  int32_t* queue_meta;      // ws [24]: queue offsets, counts, counters per XCD
  int32_t sched_P, sched_R, sched_units;
  int32_t group_kinds;      // bit k: the heads of kind k in a KV group share units, interleaved per block
  // exact slash pairs (slash_tile == 1): per-head bitmaps from the tile stage
  int32_t slash_tile;
  const uint32_t* slash_bits;   // [B,Hq,bits_words]: bit n + kBitsPad - 1 - d set iff d in D_h
  const uint32_t* col_bits;     // [B,Hq,bits_words]: bit j + kBitsPad set iff j in C_h
  int64_t bits_words;
  // ragged batch: B sequences described by samples[B] (device); the fields
  // above that describe lists, lengths and capacities are then unused, except
  // n and nq, which hold the longest sequence's (they size the schedule and
  // split queue entries).  nullptr: B sequences of length n, lists as above.
  const SampleDesc* samples;
};

// Sequence b of an attention launch, whichever way the batch is given:
// bases of head 0 of the sequence and its sizes.  Wave-uniform.
struct SampleView {
  int n, nq;
  int64_t q0, kv0;         // first row of head 0 in Q, O and lse; in K and V
  const int32_t* chunk_lo;
  const int32_t* chunk_hi;
  const int32_t* chunk_cnt;
  const int32_t* cols;
  const int32_t* col_cnt;
  const int32_t* blk_idx;
  const int32_t* blk_cnt;
  const uint32_t* slash_bits;
  const uint32_t* col_bits;
  const int32_t* tail_x;
  const int32_t* pk_cnt;
  int64_t max_chunks, max_v, max_kb, bits_words, max_tail;
};
__device__ __forceinline__ SampleView sample_view(const AttnParams& P, int b) {
  SampleView v;
  if (P.samples) {
    const SampleDesc* d = P.samples + b;
    v.n = d->n; v.nq = d->nq;
    v.q0 = d->q_row; v.kv0 = d->kv_row;
    v.chunk_lo = d->chunk_lo; v.chunk_hi = d->chunk_hi; v.chunk_cnt = d->chunk_cnt;
    v.cols = d->cols; v.col_cnt = d->col_cnt; v.blk_idx = d->blk_idx; v.blk_cnt = d->blk_cnt;
    v.slash_bits = d->slash_bits; v.col_bits = d->col_bits;
    v.tail_x = d->tail_x; v.pk_cnt = d->pk_cnt;
    v.max_chunks = d->max_chunks; v.max_v = d->max_v; v.max_kb = d->max_kb; v.bits_words = d->bits_words;
    v.max_tail = d->max_tail;
  } else {
    const int64_t bq = (int64_t)b * P.Hq;
    v.n = P.n; v.nq = P.nq;
    v.q0 = bq * (int64_t)P.n;
    v.kv0 = (int64_t)b * P.Hkv * (int64_t)P.n;
    v.chunk_lo = P.chunk_lo ? P.chunk_lo + bq * P.max_chunks : nullptr;
    v.chunk_hi = P.chunk_hi ? P.chunk_hi + bq * P.max_chunks : nullptr;
    v.chunk_cnt = P.chunk_cnt ? P.chunk_cnt + bq * P.nq : nullptr;
    v.cols = P.cols ? P.cols + bq * P.nq * P.max_v : nullptr;
    v.col_cnt = P.col_cnt ? P.col_cnt + bq * P.nq : nullptr;
    v.blk_idx = P.blk_idx ? P.blk_idx + bq * P.nq * P.max_kb : nullptr;
    v.blk_cnt = P.blk_cnt ? P.blk_cnt + bq * P.nq : nullptr;
    v.slash_bits = P.slash_bits ? P.slash_bits + bq * P.bits_words : nullptr;
    v.col_bits = P.col_bits ? P.col_bits + bq * P.bits_words : nullptr;
    v.tail_x = P.tail_x ? P.tail_x + bq * P.max_tail : nullptr;
    v.pk_cnt = P.pk_cnt ? P.pk_cnt + bq * P.nq : nullptr;
    v.max_chunks = P.max_chunks; v.max_v = P.max_v; v.max_kb = P.max_kb; v.bits_words = P.bits_words;
    v.max_tail = P.max_tail;
  }
  return v;
}
// Units of the bf16 attention schedule: each head's query blocks are cut
// into P runs of R consecutive blocks.  About kUnitsPerGroup units per KV
// group, so that one group's work spreads evenly over the eight XCD queues
// and every XCD works on the same group at about the same time (that group's
// K and V then stay in the memory-side cache); but runs of at least
// kMinRun blocks, so that the work-groups running together on one XCD
// (4 per CU, 32 CUs) mostly work on neighbouring blocks of one head; and at
// most kMaxUnits units in all.
constexpr int kUnitsPerGroup = 16;
// Pattern kinds whose heads of one KV group are scheduled together,
// interleaved per query block (they share K and V, and their key sets
// largely coincide): Block-Sparse heads always; Vertical-Slash and A-shape
// heads beyond kGroupAllMinN tokens, where the kernel is bound by memory
// traffic and the shared K/V rows count most (measured: 7% faster at 1M; at
// 32K and 128K 11% and 22% slower than runs of one head's blocks, whose
// neighbouring blocks share keys).
constexpr int kGroupAllMinN = 1 << 18;
inline int group_kinds(int n) {
  return (1 << MINF_BSPARSE) | (n > kGroupAllMinN ? (1 << MINF_VSLASH) | (1 << MINF_ASHAPE) : 0);
}
constexpr int kMinRun = 128;
constexpr int kMaxUnits = 4096;
inline void attn_sched_shape(int B, int Hq, int Hkv, int64_t nq, int* P, int* R) {
  const int bh = B * Hq;
  const int g = Hq / Hkv;
  int64_t parts = (kUnitsPerGroup + g - 1) / g;
  if (parts > nq / kMinRun) parts = nq / kMinRun;
  if (parts * bh > kMaxUnits) parts = kMaxUnits / bh;
  if (parts < 1) parts = 1;
  *P = (int)parts;
  *R = (int)((nq + parts - 1) / parts);
}
hipError_t launch_attn(const AttnParams& p, int in_bf16, int dh, hipStream_t st);
// bf16 inputs with dh = 128 (attn_bf16.hip)
hipError_t launch_attn_bf16_d128(const AttnParams& p, hipStream_t st);
// Records the start (end = 0) or end (end = 1) event of the main attention
// kernel on st while minf_timing_start() is in effect; a no-op otherwise.
void timing_mark(hipStream_t st, int end);
size_t attn_smem_bytes(int dh);

// ---------------------------------------------------------------- tiles
struct TileParams {
  const int32_t* vert_idx;   // [B,Hq,max_v]
  const int32_t* slash_idx;  // [B,Hq,max_s]
  const int32_t* blk_idx;    // [B,Hq,nq,max_kb]
  const int32_t* blk_cnt;    // [B,Hq,nq]
  minf_tiles t;
  int32_t* span_cum;         // ws [B,Hq,max_s+1]: covered offsets >= 0 before range r
  int32_t* range_chunks;     // ws [B,Hq,max_s+1]: chunks before range r
  int32_t* range_tails;      // ws [B,Hq,max_s+1]: tail-list entries before range r
  uint32_t* bitmap;          // ws [B,Hq,bm_words]: bit x+63 set iff x in S
  int32_t* head_ok;          // ws [B,Hq]
  int64_t max_v, max_s, max_kb, max_chunks, bm_words, max_tail;
  int64_t bits_words;        // words of t.slash_bits / t.col_bits (slash_tile == 1)
  int32_t slash_tile;
  int32_t B, Hq, n, nq;
  HeadTable ht;              // ASHAPE: a = sink, b = window; VSLASH: b = #columns, c = #offsets
};
hipError_t launch_tiles(const TileParams& p, bool has_vs, bool has_bs, hipStream_t st);

// ---------------------------------------------------------------- VS index
constexpr int kVsWaveKeys = 256;                  // keys per wave in the proxy passes
constexpr int kVsGroupKeys = 4 * kVsWaveKeys;     // keys per work-group
constexpr int kVsDiagSlots = kVsWaveKeys + 64;    // diagonal partials per wave

constexpr int kTopkSeg = 8192;                    // array elements per top-k work-group
struct VsWs {
  size_t part_m, part_l, lse2, cbuf, rbuf, dpart;
  size_t sync;                                    // work ticket and per-head counters of the single-launch proxy
  size_t tk_state, tk_hist, tk_cnt;               // multi-work-group top-k of c and r
  size_t total;
  int64_t nslots;                                 // proxy waves per head
  int64_t tk_segs;                                // segments of an n-element array
};
VsWs vs_workspace(int B, int Hq, int n, int nq);

struct VsParams {
  const void* Q;
  const void* K;
  int32_t* vert_idx;
  int32_t* slash_idx;
  float* vert_score;
  float* slash_score;
  int64_t max_v, max_s;
  int32_t B, Hq, Hkv, n, dh, in_bf16;
  float c;          // scale * log2(e)
  HeadTable ht;     // VSLASH: a = last_q, b = #columns, c = #offsets
  VsWs ws;
  char* ws_base;
  int32_t* status;  // minf_vs_index_fused: MINF_DEV_WAIT_EXHAUSTED when a bounded wait runs out
};
hipError_t launch_vs_index(const VsParams& p, hipStream_t st);
hipError_t launch_vs_index_fused(const VsParams& p, hipStream_t st);   // the proxy in one launch

// ---------------------------------------------------------------- BS index
struct BsParams {
  const void* Q;
  const void* K;
  int32_t* blk_idx;
  int32_t* blk_cnt;
  float* qbar;      // ws [B,Hq,nq,dh]
  uint16_t* kbar3;  // ws [B,Hkv,nq,3,dh]: each pooled key row as three bf16 terms (hi, mid, lo)
  float* scores;    // ws [heads in batch, nq, nq]
  int64_t score_heads;   // heads whose score matrices fit the workspace at once
  int64_t max_kb;
  int32_t B, Hq, Hkv, n, dh, nq, in_bf16;
  float scale;
  HeadTable ht;     // BSPARSE: a = k_b (clipped to nq), b = force flags
};
hipError_t launch_bs_index(const BsParams& p, hipStream_t st);

// Per-head fp64 sums of squared difference and squared reference over
// `heads` blocks of `per_head` elements (error.hip).
hipError_t launch_output_error(const void* O, const void* R, int64_t heads, int64_t per_head, bool bf16, double* err,
                               hipStream_t st);
// p[0 .. n) = v, a plain kernel (no memset node when a caller captures a
// graph) (error.hip).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);
// Per-head fp64 sum over n rows of exp(lse - lse_ref) (error.hip).
hipError_t launch_captured_mass(const float* lse, const float* lse_ref, int64_t heads, int64_t n, double* mass,
                                hipStream_t st);

}  // namespace minf
