/*
 * minf.h - C interface of libminf, MInference-style dynamic-sparse causal
 * attention prefill for AMD Instinct MI355X (gfx950).
 *
 * The method (PaperTrace 2.1.2 "MInference: 按 head 模式加速长上下文 Prefill",
 * sections 1-3; blog-zz7 "LLM模型之MInference", section 2.3): every query head
 * of a layer has a fixed pattern kind chosen offline (A-shape, Vertical-Slash
 * or Block-Sparse); for each input, an online index step picks the head's
 * vertical columns and slash offsets (Vertical-Slash) or key blocks
 * (Block-Sparse); the indices are turned into per-query-block tile lists; and
 * exact online-softmax attention is computed over the selected tiles only.
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout.  Q is [B, Hq, n, dh], K and V are [B, Hkv, n, dh], O is
 *   [B, Hq, n, dh]; all contiguous, row-major, no strides (section 5.1 of
 *   the MInference page: layouts are unified and contiguous before a kernel
 *   reads them).  Query head h reads KV head h / (Hq / Hkv) (GQA, same
 *   section).  Index arrays are int32, row-major, in the shapes given below.
 * Memory.  Every tensor argument is a DEVICE pointer owned by the caller and
 *   must stay valid until the work queued on `stream` has finished.  The
 *   problem and head-table structs are HOST memory, read only during the
 *   call.  The library allocates no device memory, copies nothing between
 *   host and device, and never synchronises the host: every call only queues
 *   kernels on `stream` (a hipStream_t; NULL is the default stream), so the
 *   whole path runs without a CPU round trip (section 3.1 of the page).
 * Kinds.  Each call touches only the heads of its own kind and leaves the
 *   output slots of other heads untouched.
 * Errors.  Arguments are validated before anything is queued; on failure
 *   the call returns a status, queues nothing, and minf_last_error() gives a
 *   message.  A failed kernel launch returns MINF_EHIP.  Data-dependent
 *   faults found on the device (an index out of range, unsorted or
 *   duplicated indices) set bits in `tiles->status` instead; callers read
 *   that word after their own synchronisation.  Nothing is silently
 *   truncated.
 * Threads.  The library holds no state besides a thread-local error string;
 *   calls are re-entrant.  Calls on one stream run in call order.
 */
#ifndef MINF_H
#define MINF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MINF_OK = 0,
  MINF_EINVAL = 1,         /* malformed shapes, pointers or head table          */
  MINF_EUNSUPPORTED = 2,   /* valid request the library does not implement     */
  MINF_EWORKSPACE = 3,     /* workspace smaller than minf_query_sizes() asks    */
  MINF_ECAPACITY = 4,      /* an output buffer capacity is too small            */
  MINF_EHIP = 5            /* a HIP launch failed                               */
} minf_status;

typedef enum { MINF_F32 = 0, MINF_BF16 = 1 } minf_dtype;

/* Pattern kinds (MInference page, section 2; the offline table names them
 * stream_llm, vertical_and_slash and block_sparse). */
typedef enum { MINF_ASHAPE = 0, MINF_VSLASH = 1, MINF_BSPARSE = 2 } minf_kind;

enum { MINF_FORCE_FIRST_BLOCK = 1, MINF_FORCE_DIAG_BLOCK = 2 };
enum { MINF_MAX_HEADS = 64, MINF_BLOCK = 64, MINF_MAX_LAST_Q = 64, MINF_CHUNK = 32 };
/* Offset that pads the tail list of minf_tiles: 64u - MINF_TAIL_PAD is
 * negative for every block, so a padding entry covers no key. */
enum { MINF_TAIL_PAD = 1 << 30 };

/* One query head's entry in the layer's pattern table (MInference page,
 * section 6.3: pattern kind, vertical count, slash count, block count,
 * local window and initial tokens).  Fields a kind does not use are ignored.
 *   ASHAPE : sink (g >= 0 initial keys), window (w >= 0).  Eq. 3:
 *            N(i) = [0, min(g-1, i)] U [max(0, i-w+1), i].
 *   VSLASH : last_q (1..64 sampled final rows), n_vertical (v >= 0 columns),
 *            n_slash (s >= 0 offsets).  Eq. 5 with slash expansion.
 *   BSPARSE: topk_blocks (k_b >= 1 key blocks per query block), force_flags
 *            (MINF_FORCE_FIRST_BLOCK / MINF_FORCE_DIAG_BLOCK give those
 *            blocks an infinite score, so they take budget slots).  Eq. 6. */
typedef struct {
  int32_t kind;
  int32_t sink, window;
  int32_t last_q, n_vertical, n_slash;
  int32_t topk_blocks, force_flags;
} minf_head_cfg;

/* Problem shape.  Constraints: B >= 1; 1 <= Hq <= 64; Hkv >= 1 and
 * Hq % Hkv == 0; n >= 1; dh in {64, 128}; in_dtype F32 or BF16 (Q, K and V
 * share it); out_dtype F32 or BF16; scale > 0 or 0 for 1/sqrt(dh);
 * block == 64; slash_tile == 64 or 1.  slash_tile == 64: each slash offset
 * d covers, for query block u, the keys [64u - d, 64u + 63 - d] (the 64x64
 * physical tile of section 2.1 of the MInference page).  slash_tile == 1:
 * the logical pairs of Eq. 5, i.e. key j is kept for row i iff i - j is a
 * selected offset or j a selected column (and j <= i); the tile lists are
 * the same, and the attention tests each pair against two per-head bitmaps
 * that minf_build_tiles writes (minf_tiles.slash_bits / col_bits). */
typedef struct {
  int32_t B, Hq, Hkv, n, dh;
  int32_t in_dtype;
  int32_t out_dtype;
  float scale;
  int32_t block;
  int32_t slash_tile;
} minf_problem;

/* Sizes the caller needs to allocate (all element counts except ws_bytes). */
typedef struct {
  int64_t nq;          /* query blocks ceil(n / 64)                                  */
  int64_t max_v;       /* columns per VS head: max over VS heads of min(v, n)        */
  int64_t max_s;       /* offsets per VS head: max over VS heads of min(s, n)        */
  int64_t max_kb;      /* key blocks per BS query block: max of min(k_b, nq)         */
  int64_t max_chunks;  /* slash-span chunks per VS head                              */
  int64_t ws_bytes;    /* workspace bytes that suffice for every call below          */
  int64_t bits_words;  /* 32-bit words of each per-head bitmap of minf_tiles when
                          slash_tile == 1 and the layer has a VS head, else 0      */
  int64_t max_tail;    /* entries of each per-head tail list of minf_tiles (a
                          multiple of 32)                                          */
} minf_sizes;

/* Tile lists produced by minf_build_tiles and read by minf_sparse_attn.
 * All DEVICE buffers, caller-owned, sized from minf_sizes:
 *   span_lo, span_hi  [B, Hq, max_s]      merged slash ranges in OFFSET space:
 *                     the union over d in D_h of [d-63, d], as disjoint,
 *                     non-adjacent ranges, ascending.  Key j of query block u
 *                     is slash-covered iff 64u - j lies in one of them, so one
 *                     list serves every query block.
 *   span_cnt          [B, Hq]             number of ranges.
 *   chunk_lo, chunk_hi [B, Hq, max_chunks] the whole 32-offset pieces of the
 *                     ranges, each range cut from its low end
 *                     (chunk_hi - chunk_lo = 31), ascending.  For block u a
 *                     chunk covers the 32 contiguous keys
 *                     [64u - chunk_hi, 64u - chunk_lo].  Under slash_tile == 1
 *                     a range's last, shorter piece is listed here too
 *                     (chunk_hi - chunk_lo <= 31) and the tail list is empty.
 *   chunk_cnt         [B, Hq, nq]         chunks of block u: those whose
 *                     chunk_lo <= 64u (the others lie before key 0).
 *   tail_x            [B, Hq, max_tail]   the offsets x of every range's last
 *                     piece shorter than 32, all ranges together, ascending;
 *                     entries from tail_cnt up to the next multiple of 32 hold
 *                     MINF_TAIL_PAD (they cover no key).  Entries 32c ..
 *                     32c+31 form packed chunk c: for block u its keys are
 *                     64u - x (the same for every row of the block), so the
 *                     list, like the chunk list, serves every query block.
 *   tail_cnt          [B, Hq]             entries of tail_x in use (before
 *                     the padding).
 *   pk_cnt            [B, Hq, nq]         packed chunks of block u: those
 *                     whose first entry tail_x[32c] <= 64u.
 *   cols              [B, Hq, nq, max_v]  for block u, the selected vertical
 *                     columns j <= min(64u+63, n-1) NOT covered by a slash
 *                     span of block u, ascending (MInference page section 4.1:
 *                     a vertical inside a selected range is dropped from the
 *                     column list so no pair is counted twice).
 *   col_cnt           [B, Hq, nq]
 *   kept_edges        [B, Hq] int64       E_h = sum_i |N_h(i)|, exact, for every
 *                     head (A-shape in closed form), under the problem's
 *                     slash_tile.
 *   status            [1]                 OR of MINF_DEV_* bits; the caller
 *                     zeroes it before the first call.
 *   slash_bits, col_bits [B, Hq, bits_words] uint32, only for slash_tile == 1
 *                     (else may be NULL): bit n + 127 - d of slash_bits is set
 *                     iff d is a selected offset, bit j + 128 of col_bits iff
 *                     j is a selected column (bit b is bit b%32 of word b/32;
 *                     the other bits are zero). */
typedef struct {
  int32_t* span_lo;
  int32_t* span_hi;
  int32_t* span_cnt;
  int32_t* chunk_lo;
  int32_t* chunk_hi;
  int32_t* chunk_cnt;
  int32_t* cols;
  int32_t* col_cnt;
  int64_t* kept_edges;
  int32_t* status;
  uint32_t* slash_bits;
  uint32_t* col_bits;
  int32_t* tail_x;
  int32_t* tail_cnt;
  int32_t* pk_cnt;
} minf_tiles;

enum {
  MINF_DEV_BAD_VERTICAL = 1,   /* a column index outside [0, n) or not ascending  */
  MINF_DEV_BAD_SLASH = 2,      /* an offset outside [0, n) or not ascending       */
  MINF_DEV_BAD_BLOCK = 4,      /* a block index outside [0, u] or not ascending   */
  MINF_DEV_CAPACITY = 8,       /* a list outgrew the capacity it was sized with   */
  MINF_DEV_WAIT_EXHAUSTED = 16 /* minf_vs_index_fused: a bounded wait ran out     */
};

/* Fills *out for the given problem and head table (host only, no GPU work).
 * Validates the problem exactly as the calls below do. */
minf_status minf_query_sizes(const minf_problem* prob, const minf_head_cfg* heads,
                             minf_sizes* out);

/* Vertical-Slash index estimation (MInference page, section 6.2; blog
 * section 2.3.2, step 1-2 of the Vertical-Slash estimate).  For every VS head
 * h (for each batch b): with R the last min(last_q, n) rows, the proxy weights
 * are the causal softmax over keys j <= i of scale * q_i . k_j for i in R;
 *   c_j = sum_{i in R} weight(i, j),    r_d = sum_{i in R} weight(i, i - d).
 * The top n_vertical columns of c and the top n_slash offsets of r are kept
 * (order: score descending, then index ascending) and written ascending:
 *   vert_idx  [B, Hq, max_v]  columns; entries past min(v, n) are -1
 *   slash_idx [B, Hq, max_s]  offsets d; entries past min(s, n) are -1
 *   vert_score, slash_score   [B, Hq, n] fp32 c and r, or NULL to skip.
 * Q, K: in_dtype.  ws: DEVICE workspace of at least ws_bytes. */
minf_status minf_vs_index(const minf_problem* prob, const minf_head_cfg* heads,
                          const void* Q, const void* K,
                          int32_t* vert_idx, int32_t* slash_idx,
                          float* vert_score, float* slash_score,
                          void* ws, size_t ws_bytes, void* stream);

/* The same Vertical-Slash estimation with the proxy in one launch (MInference
 * page, section 3.1: on a GPU the index cost is counted in read and write
 * rounds and synchronisations, so fusing the reduce with the selection
 * matters): the
 * per-row LSE fold and the column and slash sums run in the same grid as the
 * proxy scores, a work-group of the second pass waiting (bounded) for its
 * head's LSE.  Arguments, outputs, workspace and errors as minf_vs_index;
 * scores equal minf_vs_index's up to the summation order of the LSE and slash
 * sums, so selections can differ only between near-equal scores.  The
 * waits end by construction (a second-pass work-group waits only for work
 * that started before it and waits for nothing); each is still bounded (about
 * a second).  A wait that ran out sets MINF_DEV_WAIT_EXHAUSTED in *status
 * (DEVICE int32, required, OR-ed into; the caller zeroes it first) and
 * leaves zero column and slash scores for its key range, so the selections
 * of that call are not to be used.  The two-launch minf_vs_index is faster
 * on MI355X and remains the path that minf_prefill_ragged and the layer use. */
minf_status minf_vs_index_fused(const minf_problem* prob, const minf_head_cfg* heads,
                                const void* Q, const void* K,
                                int32_t* vert_idx, int32_t* slash_idx,
                                float* vert_score, float* slash_score,
                                void* ws, size_t ws_bytes, int32_t* status, void* stream);

/* Block-Sparse index estimation (MInference page, section 2, Eq. 6 and the
 * mean-pooling proxy; blog section 2.3.2).  For every BS head: Q and K are
 * mean-pooled over 64-row blocks (the last block over its true length),
 * r_uv = scale * Qbar_u . Kbar_v for v <= u in fp32, forced blocks get +inf,
 * and J_u is the top min(k_b, u+1) of row u (score descending, index
 * ascending), written ascending:
 *   blk_idx [B, Hq, nq, max_kb]  (entries past blk_cnt are -1)
 *   blk_cnt [B, Hq, nq]. */
minf_status minf_bs_index(const minf_problem* prob, const minf_head_cfg* heads,
                          const void* Q, const void* K,
                          int32_t* blk_idx, int32_t* blk_cnt,
                          void* ws, size_t ws_bytes, void* stream);

/* Index -> tile lists (MInference page section 4.1 / blog section 2.3.3,
 * "get Vertical-Slash index": sort, merge the slash ranges, drop covered
 * verticals, emit counts and indices).  Reads vert_idx / slash_idx of the VS
 * heads and blk_idx / blk_cnt of the BS heads (either pair may be NULL when
 * the layer has no head of that kind), checks them, and fills *tiles
 * (including kept_edges for every head).  Invalid indices set status bits. */
minf_status minf_build_tiles(const minf_problem* prob, const minf_head_cfg* heads,
                             const int32_t* vert_idx, const int32_t* slash_idx,
                             const int32_t* blk_idx, const int32_t* blk_cnt,
                             const minf_tiles* tiles,
                             void* ws, size_t ws_bytes, void* stream);

/* Sparse attention over the selected tiles (MInference page sections 1.1 and
 * 3.2, Eq. 2 restricted to N_h(i), merged tile by tile with the running
 * max / sum / accumulator of Eq. 7-8; blog section 2.3.3).  For every head:
 *   o_i = sum_{j in N_h(i)} softmax_j(scale * q_i . k_j) v_j,
 * with N_h(i) from Eq. 3 (A-shape), the tile lists (VS) or blk_idx (BS).
 * Excluded pairs never enter the maximum or the sum.  A row with no
 * candidate gets o = 0 and lse = -inf.
 *   O   [B, Hq, n, dh] in out_dtype
 *   lse [B, Hq, n] fp32 natural-log sum of exp of the kept scores, or NULL.
 * bf16 inputs: products exact, fp32 accumulation, probabilities rounded to
 * bf16 for the P.V product.  fp32 inputs: fp32 throughout. */
minf_status minf_sparse_attn(const minf_problem* prob, const minf_head_cfg* heads,
                             const void* Q, const void* K, const void* V,
                             const int32_t* blk_idx, const int32_t* blk_cnt,
                             const minf_tiles* tiles,
                             void* O, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* minf_sparse_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * minf_sparse_attn, minus ws / ws_bytes: the attention scheduler's scratch
 * (unit costs and order, XCD assignment, the item queue and its counters)
 * lives in a file-scope device array of the library, 8 MiB per device, held
 * until the process ends.  A problem whose scheduler needs more (about 2M
 * (batch, head, query block) items, e.g. B * Hq * ceil(n / 64) > 2 million)
 * is refused with MINF_EWORKSPACE before anything is queued.  The call
 * allocates nothing; it looks up the array's address on the current device
 * the first time it runs there (the stream must belong to the current
 * device).  Every call on one device shares that device's array, and the
 * scheduler rewrites all of it on each call (nothing needs clearing between
 * calls), so calls that overlap in time on one device -- on different
 * streams or from several threads -- race: order them on one stream. */
minf_status minf_sparse_attn_static(const minf_problem* prob, const minf_head_cfg* heads,
                                    const void* Q, const void* K, const void* V,
                                    const int32_t* blk_idx, const int32_t* blk_cnt,
                                    const minf_tiles* tiles, void* O, float* lse, void* stream);

/* Per-head output error, for the offline kernel-aware pattern search
 * (MInference page sections 3.1 and 6.3; blog section 2.3.1, Eq. 2: each
 * candidate pattern's attention is compared with dense attention on a
 * calibration input).  For every (b, h), with O and O_ref [B, Hq, n, dh] in
 * the problem's out_dtype (device memory, read only):
 *   err[2 (b Hq + h)]     = sum over rows and columns of (O - O_ref)^2,
 *   err[2 (b Hq + h) + 1] = sum of O_ref^2,
 * accumulated in fp64 in a fixed order (two runs give identical bits).
 * err: device memory of 2 B Hq doubles, written.  Only B, Hq, n, dh and
 * out_dtype of *prob are read; the head table is not needed.  MINF_EINVAL
 * for null pointers or bad sizes, MINF_EUNSUPPORTED for dh not 64 or 128. */
minf_status minf_output_error(const minf_problem* prob, const void* O, const void* O_ref, double* err, void* stream);

/* Captured attention mass, for the same search (MInference page section
 * 3.1, "covered attention mass"; blog section 2.3.1, Eq. 2): a row whose
 * kept keys carry the fraction m of the dense softmax has
 * m = exp(lse - lse_ref), with lse from minf_sparse_attn for the candidate
 * and lse_ref for dense attention, and Eq. 2's L1 distance between the
 * renormalised and the dense attention row is 2 (1 - m).  For every (b, h):
 *   mass[b Hq + h] = sum over the n rows of exp(lse - lse_ref)
 * (rows with lse = -inf, i.e. no kept key, add 0), fp64, fixed order.
 * lse, lse_ref: device [B, Hq, n] fp32, read only; mass: device, B Hq
 * doubles, written.  Only B, Hq and n of *prob are read.  MINF_EINVAL for
 * null pointers or bad sizes. */
minf_status minf_captured_mass(const minf_problem* prob, const float* lse, const float* lse_ref, double* mass,
                               void* stream);

/* Ragged (variable-length) batch prefill: prob->B sequences of lengths
 * seq_lens[b] (host array, each in [1, prob->n]), packed back to back with
 * no padding (the serving case of the cost-model page, section 2.2: a batch
 * padded to its longest request spends projection and attention work on the
 * padding).  Sample b is the contiguous block at token offset
 * t_b = sum_{c<b} seq_lens[c]:
 *   Q, O: [Hq, len_b, dh] at element offset Hq*dh*t_b (input / output type),
 *   K, V: [Hkv, len_b, dh] at element offset Hkv*dh*t_b,
 *   lse:  [Hq, len_b] at offset Hq*t_b (fp32; NULL to skip),
 * so the full tensors hold Hq*dh*sum(len) (resp. Hkv*dh*sum(len)) elements.
 * The index and tile stages (minf_vs_index, minf_bs_index,
 * minf_build_tiles) run for each sample as a problem of its own length with
 * B = 1, one after another on `stream`; then the sparse attention of every
 * sample runs in ONE launch, whose work items (sample, head, query block)
 * are scheduled together.  Indices are per sample, and no window, slash or
 * block crosses a sample boundary.
 *   kept_edges: device [B, Hq] int64, E_h of each sample and head, or NULL;
 *   status: device int32[1], zeroed by the call, then the OR of MINF_DEV_*
 *     bits over all samples;
 *   ws: device workspace of at least minf_ragged_ws_bytes(prob, heads,
 *     seq_lens) bytes: every sample's index and tile buffers, one stage
 *     workspace the samples reuse in turn, the batch's attention schedule
 *     and a table of per-sample descriptors.
 * Errors as for the four calls; MINF_EINVAL for a null seq_lens or a length
 * outside [1, n]. */
minf_status minf_ragged_ws_bytes(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* seq_lens,
                                 int64_t* ws_bytes);
minf_status minf_prefill_ragged(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* seq_lens,
                                const void* Q, const void* K, const void* V, void* O, float* lse,
                                int64_t* kept_edges, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* Kernel timing, for measurement harnesses; computing never needs it.
 * After minf_timing_start(max_calls), each of the next max_calls calls of
 * minf_sparse_attn records a HIP event pair on its stream around its main
 * attention kernel only (the work-item scheduling kernels before it are
 * outside the pair).  Later calls record nothing.  The library owns the
 * events: start creates them (replacing any from an earlier start, unread),
 * read releases them.  max_calls must lie in [1, 65536] (else MINF_EINVAL);
 * MINF_EHIP if an event cannot be created.
 * minf_timing_read waits on the host for the recorded pairs, writes the
 * first min(recorded, cap) durations in milliseconds to ms[] (host memory),
 * sets *count to the number of recorded pairs and ends the timing.  Not
 * thread safe: one timing at a time per process. */
minf_status minf_timing_start(int32_t max_calls);
minf_status minf_timing_read(float* ms, int32_t cap, int32_t* count);

const char* minf_status_string(minf_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* minf_last_error(void);
/* Library version string. */
const char* minf_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MINF_H */
