// Host side of the C interface declared in include/minf.h: argument checks,
// size queries, workspace layout and kernel launches.  No device memory is
// allocated and the host never waits on the GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

minf_status fail(minf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// A Block-Sparse row's selection keeps the row's scores in the registers of
// one work-group (256 threads x 128 scores), so a row holds at most this many
// key blocks.
constexpr int64_t kBsMaxBlocks = 256 * 128;

struct Derived {
  int64_t nq = 0, max_v = 0, max_s = 0, max_kb = 0, max_chunks = 0, bm_words = 0, bits_words = 0, max_tail = 0;
  bool has_a = false, has_vs = false, has_bs = false;
  int hq_vs = 0, hq_bs = 0;
  minf::HeadTable ht{};
  float scale = 0.f;
};

minf_status validate(const minf_problem* p, const minf_head_cfg* heads, Derived* d) {
  g_err[0] = 0;
  if (!p || !heads) return fail(MINF_EINVAL, "null problem or head table");
  if (p->B < 1 || p->n < 1) return fail(MINF_EINVAL, "B and n must be >= 1 (B=%d n=%d)", p->B, p->n);
  if (p->Hq < 1 || p->Hq > MINF_MAX_HEADS) return fail(MINF_EINVAL, "Hq must be in [1, %d] (Hq=%d)", MINF_MAX_HEADS, p->Hq);
  if (p->Hkv < 1 || p->Hq % p->Hkv != 0) return fail(MINF_EINVAL, "Hq %% Hkv must be 0 (Hq=%d Hkv=%d)", p->Hq, p->Hkv);
  if (p->dh != 64 && p->dh != 128) return fail(MINF_EUNSUPPORTED, "dh must be 64 or 128 (dh=%d)", p->dh);
  if (p->in_dtype != MINF_F32 && p->in_dtype != MINF_BF16) return fail(MINF_EINVAL, "bad in_dtype %d", p->in_dtype);
  if (p->out_dtype != MINF_F32 && p->out_dtype != MINF_BF16) return fail(MINF_EINVAL, "bad out_dtype %d", p->out_dtype);
  if (!(p->scale >= 0.f) || isinf(p->scale)) return fail(MINF_EINVAL, "scale must be finite and >= 0");
  if (p->block != MINF_BLOCK) return fail(MINF_EUNSUPPORTED, "block must be %d (block=%d)", MINF_BLOCK, p->block);
  if (p->slash_tile != 64 && p->slash_tile != 1)
    return fail(MINF_EINVAL, "slash_tile must be 64 or 1 (slash_tile=%d)", p->slash_tile);
  if ((int64_t)p->B * p->Hq * p->n * p->dh > ((int64_t)1 << 40)) return fail(MINF_EINVAL, "problem too large");
  d->nq = (p->n + MINF_BLOCK - 1) / MINF_BLOCK;
  d->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->dh);
  int64_t mv = 0, ms = 0, mk = 0;
  for (int h = 0; h < p->Hq; ++h) {
    const minf_head_cfg& c = heads[h];
    d->ht.kind[h] = c.kind;
    switch (c.kind) {
      case MINF_ASHAPE:
        if (c.sink < 0 || c.window < 0) return fail(MINF_EINVAL, "head %d: A-shape sink/window must be >= 0", h);
        d->ht.a[h] = (int32_t)std::min<int64_t>(c.sink, p->n);
        d->ht.b[h] = (int32_t)std::min<int64_t>(c.window, p->n);
        d->has_a = true;
        break;
      case MINF_VSLASH: {
        if (c.last_q < 1 || c.last_q > MINF_MAX_LAST_Q)
          return fail(c.last_q > MINF_MAX_LAST_Q ? MINF_EUNSUPPORTED : MINF_EINVAL,
                      "head %d: last_q must be in [1, %d] (last_q=%d)", h, MINF_MAX_LAST_Q, c.last_q);
        if (c.n_vertical < 0 || c.n_slash < 0) return fail(MINF_EINVAL, "head %d: negative VS budget", h);
        const int64_t v = std::min<int64_t>(c.n_vertical, p->n), s = std::min<int64_t>(c.n_slash, p->n);
        d->ht.a[h] = c.last_q;
        d->ht.b[h] = (int32_t)v;
        d->ht.c[h] = (int32_t)s;
        mv = std::max(mv, v);
        ms = std::max(ms, s);
        d->has_vs = true;
        d->hq_vs++;
        break;
      }
      case MINF_BSPARSE: {
        if (c.topk_blocks < 1) return fail(MINF_EINVAL, "head %d: topk_blocks must be >= 1", h);
        if (c.force_flags & ~(MINF_FORCE_FIRST_BLOCK | MINF_FORCE_DIAG_BLOCK))
          return fail(MINF_EINVAL, "head %d: unknown force flags 0x%x", h, c.force_flags);
        if (d->nq > kBsMaxBlocks)
          return fail(MINF_EUNSUPPORTED, "head %d: Block-Sparse rows of more than %lld blocks (n > %lld) are not supported",
                      h, (long long)kBsMaxBlocks, (long long)kBsMaxBlocks * MINF_BLOCK);
        const int64_t k = std::min<int64_t>(c.topk_blocks, d->nq);
        d->ht.a[h] = (int32_t)k;
        d->ht.b[h] = c.force_flags;
        mk = std::max(mk, k);
        d->has_bs = true;
        d->hq_bs++;
        break;
      }
      default:
        return fail(MINF_EINVAL, "head %d: unknown pattern kind %d", h, c.kind);
    }
  }
  d->max_v = round_up(mv, MINF_CHUNK);
  d->max_s = std::max<int64_t>(ms, 1);
  d->max_kb = std::max<int64_t>(mk, 1);
  d->max_chunks = (p->n + 63 + 31) / 32 + d->max_s + 1;
  d->bm_words = (p->n + 63 + 31) / 32;
  d->bits_words = (p->slash_tile == 1 && d->has_vs) ? minf::exact_bits_words(p->n) : 0;
  // every range leaves a tail of at most 31 offsets, and the tails are
  // disjoint offsets in [-63, n); padded to whole packed chunks
  d->max_tail = round_up(std::min<int64_t>(31 * d->max_s, (int64_t)p->n + 63), MINF_CHUNK);
  return MINF_OK;
}

// ---- workspace layout (bytes, 256-aligned pieces) ----
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; }
};

struct TilesWs { size_t span_cum, range_chunks, range_tails, bitmap, head_ok, total; };
TilesWs tiles_ws(const minf_problem* p, const Derived& d) {
  Carve c;
  TilesWs w;
  const size_t BH = (size_t)p->B * p->Hq;
  w.span_cum = c.take(BH * (d.max_s + 1) * 4);
  w.range_chunks = c.take(BH * (d.max_s + 1) * 4);
  w.range_tails = c.take(BH * (d.max_s + 1) * 4);
  w.bitmap = c.take(BH * d.bm_words * 4);
  w.head_ok = c.take(BH * 4);
  w.total = c.off;
  return w;
}

// Block scores of at most this many bytes are resident at once; heads are
// processed in batches that fit.
constexpr size_t kScoreBytesCap = size_t(2) << 30;

struct BsWs { size_t qbar, kbar, scores, total; int64_t score_heads; };
BsWs bs_ws(const minf_problem* p, const Derived& d) {
  Carve c;
  BsWs w;
  w.qbar = c.take((size_t)p->B * p->Hq * d.nq * p->dh * 4);
  w.kbar = c.take((size_t)p->B * p->Hkv * d.nq * p->dh * 3 * 2);
  const size_t per_head = (size_t)d.nq * d.nq * 4;
  const int64_t heads = (int64_t)p->B * std::max(d.hq_bs, 1);
  w.score_heads = std::max<int64_t>(1, std::min<int64_t>({heads, 64, (int64_t)(kScoreBytesCap / per_head)}));
  w.scores = c.take(per_head * w.score_heads);
  w.total = c.off;
  return w;
}

minf::VsWs vs_ws(const minf_problem* p, const Derived& d) {
  return minf::vs_workspace(p->B, p->Hq, p->n, (int)d.nq);
}

struct AttnWs { size_t cost, order, uxcd, uoff, queue, meta, total; int P, R, units; };
AttnWs attn_ws(const minf_problem* p, const Derived& d) {
  Carve c;
  AttnWs w;
  minf::attn_sched_shape(p->B, p->Hq, p->Hkv, d.nq, &w.P, &w.R);
  w.units = p->B * p->Hq * w.P;
  w.cost = c.take((size_t)w.units * 8);
  w.order = c.take((size_t)w.units * 4);
  w.uxcd = c.take((size_t)w.units * 4);
  w.uoff = c.take((size_t)w.units * 4);
  w.queue = c.take((size_t)p->B * p->Hq * d.nq * 4);
  w.meta = c.take(24 * 4);
  w.total = c.off;
  return w;
}

size_t ws_total(const minf_problem* p, const Derived& d) {
  size_t t = std::max(tiles_ws(p, d).total, attn_ws(p, d).total);
  if (d.has_bs) t = std::max(t, bs_ws(p, d).total);
  if (d.has_vs) t = std::max(t, vs_ws(p, d).total);
  return std::max<size_t>(t, 256);
}

minf_status check_ws(const minf_problem* p, const Derived& d, void* ws, size_t ws_bytes) {
  const size_t need = ws_total(p, d);
  if (!ws) return fail(MINF_EWORKSPACE, "workspace pointer is null");
  if (ws_bytes < need) return fail(MINF_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  return MINF_OK;
}

minf_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MINF_OK;
  return fail(MINF_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Scratch of minf_sparse_attn_static (the attention scheduler's unit costs,
// order, XCD assignment, item queue and queue counters), a file-scope device
// array: each device the library runs on holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it stands for no device address): the address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

minf_status scratch_on_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MINF_EHIP, "minf_sparse_attn_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MINF_EUNSUPPORTED, "minf_sparse_attn_static: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MINF_EHIP, "minf_sparse_attn_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MINF_OK;
}

// Event pairs of minf_timing_start() / minf_timing_read(): pair i brackets
// the main attention kernel of the i-th minf_sparse_attn call since the start.
struct Timing {
  std::vector<hipEvent_t> ev;   // 2 * cap events: start, end, start, end, ...
  int cap = 0, used = 0;
  hipError_t err = hipSuccess;
};
Timing g_timing;

void timing_release() {
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing = Timing{};
}

}  // namespace

namespace minf {

void timing_mark(hipStream_t st, int end) {
  if (g_timing.used >= g_timing.cap) return;
  const hipError_t e = hipEventRecord(g_timing.ev[2 * g_timing.used + end], st);
  if (e != hipSuccess && g_timing.err == hipSuccess) g_timing.err = e;
  if (end) ++g_timing.used;
}

}  // namespace minf

extern "C" {

const char* minf_status_string(minf_status s) {
  switch (s) {
    case MINF_OK: return "ok";
    case MINF_EINVAL: return "invalid argument";
    case MINF_EUNSUPPORTED: return "unsupported";
    case MINF_EWORKSPACE: return "workspace too small";
    case MINF_ECAPACITY: return "capacity too small";
    case MINF_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* minf_last_error(void) { return g_err; }
const char* minf_version(void) { return "minf 0.1 gfx950"; }

minf_status minf_query_sizes(const minf_problem* prob, const minf_head_cfg* heads, minf_sizes* out) {
  Derived d;
  minf_status s = validate(prob, heads, &d);
  if (s != MINF_OK) return s;
  if (!out) return fail(MINF_EINVAL, "null output");
  out->nq = d.nq;
  out->max_v = d.max_v;
  out->max_s = d.max_s;
  out->max_kb = d.max_kb;
  out->max_chunks = d.max_chunks;
  out->ws_bytes = (int64_t)ws_total(prob, d);
  out->bits_words = d.bits_words;
  out->max_tail = d.max_tail;
  return MINF_OK;
}

static minf_status vs_index_impl(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                                 int32_t* vert_idx, int32_t* slash_idx, float* vert_score, float* slash_score,
                                 void* ws, size_t ws_bytes, int32_t* status, void* stream, bool fused) {
  Derived d;
  minf_status s = validate(prob, heads, &d);
  if (s != MINF_OK) return s;
  if (!d.has_vs) return MINF_OK;
  if (!Q || !K || !vert_idx || !slash_idx) return fail(MINF_EINVAL, "null Q, K or index output");
  if (fused && !status) return fail(MINF_EINVAL, "minf_vs_index_fused needs a status word");
  if ((s = check_ws(prob, d, ws, ws_bytes)) != MINF_OK) return s;
  minf::VsParams v{};
  v.status = status;
  v.Q = Q; v.K = K;
  v.vert_idx = vert_idx; v.slash_idx = slash_idx;
  v.vert_score = vert_score; v.slash_score = slash_score;
  v.max_v = d.max_v; v.max_s = d.max_s;
  v.B = prob->B; v.Hq = prob->Hq; v.Hkv = prob->Hkv; v.n = prob->n; v.dh = prob->dh;
  v.in_bf16 = prob->in_dtype == MINF_BF16;
  v.c = d.scale * minf::kLog2e;
  v.ht = d.ht;
  v.ws = vs_ws(prob, d);
  v.ws_base = static_cast<char*>(ws);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return fused ? hip_status(minf::launch_vs_index_fused(v, st), "minf_vs_index_fused launch")
               : hip_status(minf::launch_vs_index(v, st), "minf_vs_index launch");
}

minf_status minf_vs_index(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                          int32_t* vert_idx, int32_t* slash_idx, float* vert_score, float* slash_score,
                          void* ws, size_t ws_bytes, void* stream) {
  return vs_index_impl(prob, heads, Q, K, vert_idx, slash_idx, vert_score, slash_score, ws, ws_bytes, nullptr, stream,
                       false);
}

minf_status minf_vs_index_fused(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                                int32_t* vert_idx, int32_t* slash_idx, float* vert_score, float* slash_score,
                                void* ws, size_t ws_bytes, int32_t* status, void* stream) {
  return vs_index_impl(prob, heads, Q, K, vert_idx, slash_idx, vert_score, slash_score, ws, ws_bytes, status, stream,
                       true);
}

minf_status minf_bs_index(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                          int32_t* blk_idx, int32_t* blk_cnt, void* ws, size_t ws_bytes, void* stream) {
  Derived d;
  minf_status s = validate(prob, heads, &d);
  if (s != MINF_OK) return s;
  if (!d.has_bs) return MINF_OK;
  if (!Q || !K || !blk_idx || !blk_cnt) return fail(MINF_EINVAL, "null Q, K or index output");
  if ((s = check_ws(prob, d, ws, ws_bytes)) != MINF_OK) return s;
  const BsWs w = bs_ws(prob, d);
  minf::BsParams b{};
  b.Q = Q; b.K = K; b.blk_idx = blk_idx; b.blk_cnt = blk_cnt;
  b.qbar = reinterpret_cast<float*>(static_cast<char*>(ws) + w.qbar);
  b.kbar3 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + w.kbar);
  b.scores = reinterpret_cast<float*>(static_cast<char*>(ws) + w.scores);
  b.score_heads = w.score_heads;
  b.max_kb = d.max_kb;
  b.B = prob->B; b.Hq = prob->Hq; b.Hkv = prob->Hkv; b.n = prob->n; b.dh = prob->dh; b.nq = (int)d.nq;
  b.in_bf16 = prob->in_dtype == MINF_BF16;
  b.scale = d.scale;
  b.ht = d.ht;
  return hip_status(minf::launch_bs_index(b, static_cast<hipStream_t>(stream)), "minf_bs_index launch");
}

minf_status minf_build_tiles(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* vert_idx,
                             const int32_t* slash_idx, const int32_t* blk_idx, const int32_t* blk_cnt,
                             const minf_tiles* tiles, void* ws, size_t ws_bytes, void* stream) {
  Derived d;
  minf_status s = validate(prob, heads, &d);
  if (s != MINF_OK) return s;
  if (!tiles || !tiles->kept_edges || !tiles->status) return fail(MINF_EINVAL, "null tiles, kept_edges or status");
  if (d.has_vs && (!vert_idx || !slash_idx || !tiles->span_lo || !tiles->span_hi || !tiles->span_cnt ||
                   !tiles->chunk_lo || !tiles->chunk_hi || !tiles->chunk_cnt || !tiles->cols || !tiles->col_cnt ||
                   !tiles->tail_x || !tiles->tail_cnt || !tiles->pk_cnt))
    return fail(MINF_EINVAL, "a Vertical-Slash head needs vert_idx, slash_idx and every span/chunk/tail/column buffer");
  if (d.has_bs && (!blk_idx || !blk_cnt)) return fail(MINF_EINVAL, "a Block-Sparse head needs blk_idx and blk_cnt");
  if (d.bits_words > 0 && (!tiles->slash_bits || !tiles->col_bits))
    return fail(MINF_EINVAL, "slash_tile=1 with a Vertical-Slash head needs slash_bits and col_bits");
  if ((s = check_ws(prob, d, ws, ws_bytes)) != MINF_OK) return s;
  const TilesWs w = tiles_ws(prob, d);
  char* base = static_cast<char*>(ws);
  minf::TileParams t{};
  t.vert_idx = vert_idx; t.slash_idx = slash_idx; t.blk_idx = blk_idx; t.blk_cnt = blk_cnt;
  t.t = *tiles;
  t.span_cum = reinterpret_cast<int32_t*>(base + w.span_cum);
  t.range_chunks = reinterpret_cast<int32_t*>(base + w.range_chunks);
  t.range_tails = reinterpret_cast<int32_t*>(base + w.range_tails);
  t.bitmap = reinterpret_cast<uint32_t*>(base + w.bitmap);
  t.head_ok = reinterpret_cast<int32_t*>(base + w.head_ok);
  t.max_v = d.max_v; t.max_s = d.max_s; t.max_kb = d.max_kb; t.max_chunks = d.max_chunks; t.bm_words = d.bm_words;
  t.max_tail = d.max_tail;
  t.bits_words = d.bits_words; t.slash_tile = prob->slash_tile;
  t.B = prob->B; t.Hq = prob->Hq; t.n = prob->n; t.nq = (int)d.nq;
  t.ht = d.ht;
  return hip_status(minf::launch_tiles(t, d.has_vs, d.has_bs, static_cast<hipStream_t>(stream)),
                    "minf_build_tiles launch");
}

// Checks shared by minf_sparse_attn and minf_sparse_attn_static.
static minf_status attn_checks(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                               const void* V, const int32_t* blk_idx, const int32_t* blk_cnt, const minf_tiles* tiles,
                               void* O, Derived* d) {
  minf_status s = validate(prob, heads, d);
  if (s != MINF_OK) return s;
  if (!Q || !K || !V || !O) return fail(MINF_EINVAL, "null Q, K, V or O");
  if (d->has_bs && (!blk_idx || !blk_cnt)) return fail(MINF_EINVAL, "a Block-Sparse head needs blk_idx and blk_cnt");
  if (d->has_vs && (!tiles || !tiles->chunk_lo || !tiles->chunk_hi || !tiles->chunk_cnt || !tiles->cols ||
                    !tiles->col_cnt || !tiles->tail_x || !tiles->pk_cnt))
    return fail(MINF_EINVAL, "a Vertical-Slash head needs the tile lists from minf_build_tiles");
  if (d->bits_words > 0 && (!tiles->slash_bits || !tiles->col_bits))
    return fail(MINF_EINVAL, "slash_tile=1 with a Vertical-Slash head needs slash_bits and col_bits");
  return MINF_OK;
}

// The attention launch on a workspace `wb` that holds attn_ws(prob, d).total bytes.
// With `samples` (device, prob->B descriptors) the batch is ragged: each
// sequence's lists, length and row offsets come from its descriptor, and
// blk_idx, blk_cnt and tiles are not read.
static minf_status attn_launch(const minf_problem* prob, const Derived& d, const void* Q, const void* K, const void* V,
                               const int32_t* blk_idx, const int32_t* blk_cnt, const minf_tiles* tiles, void* O,
                               float* lse, char* wb, void* stream, const char* what,
                               const minf::SampleDesc* samples = nullptr) {
  const AttnWs w = attn_ws(prob, d);
  minf::AttnParams a{};
  a.sched_cost = reinterpret_cast<int64_t*>(wb + w.cost);
  a.sched_order = reinterpret_cast<int32_t*>(wb + w.order);
  a.unit_xcd = reinterpret_cast<int32_t*>(wb + w.uxcd);
  a.unit_off = reinterpret_cast<int32_t*>(wb + w.uoff);
  a.queue = reinterpret_cast<int32_t*>(wb + w.queue);
  a.queue_meta = reinterpret_cast<int32_t*>(wb + w.meta);
  a.sched_P = w.P; a.sched_R = w.R; a.sched_units = w.units;
  a.group_kinds = minf::group_kinds(prob->n);
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  a.blk_idx = blk_idx; a.blk_cnt = blk_cnt;
  if (d.has_vs && !samples) {
    a.chunk_lo = tiles->chunk_lo; a.chunk_hi = tiles->chunk_hi; a.chunk_cnt = tiles->chunk_cnt;
    a.cols = tiles->cols; a.col_cnt = tiles->col_cnt;
    a.tail_x = tiles->tail_x; a.pk_cnt = tiles->pk_cnt;
  }
  a.samples = samples;
  a.max_kb = d.max_kb; a.max_chunks = d.max_chunks; a.max_v = d.max_v; a.max_tail = d.max_tail;
  a.B = prob->B; a.Hq = prob->Hq; a.Hkv = prob->Hkv; a.n = prob->n; a.nq = (int)d.nq;
  a.gsz = prob->Hq / prob->Hkv;
  a.n_utiles = (int)((d.nq + 7) / 8);
  a.n_segs = prob->B * a.n_utiles * prob->Hkv;
  a.c = d.scale * minf::kLog2e;
  a.out_bf16 = prob->out_dtype == MINF_BF16;
  a.slash_tile = prob->slash_tile;
  if (d.bits_words > 0 && !samples) {
    a.slash_bits = tiles->slash_bits;
    a.col_bits = tiles->col_bits;
    a.bits_words = d.bits_words;
  }
  a.ht = d.ht;
  return hip_status(minf::launch_attn(a, prob->in_dtype == MINF_BF16, prob->dh, static_cast<hipStream_t>(stream)),
                    what);
}

minf_status minf_sparse_attn(const minf_problem* prob, const minf_head_cfg* heads, const void* Q, const void* K,
                             const void* V, const int32_t* blk_idx, const int32_t* blk_cnt, const minf_tiles* tiles,
                             void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Derived d;
  minf_status s = attn_checks(prob, heads, Q, K, V, blk_idx, blk_cnt, tiles, O, &d);
  if (s != MINF_OK) return s;
  if ((s = check_ws(prob, d, ws, ws_bytes)) != MINF_OK) return s;
  return attn_launch(prob, d, Q, K, V, blk_idx, blk_cnt, tiles, O, lse, static_cast<char*>(ws), stream,
                     "minf_sparse_attn launch");
}

minf_status minf_sparse_attn_static(const minf_problem* prob, const minf_head_cfg* heads, const void* Q,
                                    const void* K, const void* V, const int32_t* blk_idx, const int32_t* blk_cnt,
                                    const minf_tiles* tiles, void* O, float* lse, void* stream) {
  Derived d;
  minf_status s = attn_checks(prob, heads, Q, K, V, blk_idx, blk_cnt, tiles, O, &d);
  if (s != MINF_OK) return s;
  const size_t need = attn_ws(prob, d).total;
  if (need > kScratchBytes)
    return fail(MINF_EWORKSPACE, "minf_sparse_attn_static: the problem needs %zu bytes of scratch, the static scratch "
                "holds %zu (use minf_sparse_attn with a workspace)", need, kScratchBytes);
  char* wb = nullptr;
  if ((s = scratch_on_current_device(&wb)) != MINF_OK) return s;
  return attn_launch(prob, d, Q, K, V, blk_idx, blk_cnt, tiles, O, lse, wb, stream, "minf_sparse_attn_static launch");
}

// ---- ragged batches: the workspace holds every sequence's index and tile
// buffers (each laid out as for a B = 1 problem of its own length), one stage
// workspace that the sequences' index and tile stages reuse in turn, the
// attention schedule of the whole batch and the table of sequence
// descriptors that the one attention launch reads.
struct RaggedRegion {
  size_t vert, slash, blk, blkcnt, span_lo, span_hi, span_cnt, chunk_lo, chunk_hi, chunk_cnt, cols, col_cnt, sbits,
      cbits, tail_x, tail_cnt, pk_cnt;
  Derived d;
};
struct RaggedLayout {
  std::vector<RaggedRegion> r;
  minf_problem all;     // the batch as one attention problem: B sequences, n = the longest
  Derived d_all;
  size_t stage, stage_bytes, attn, table, kept, total;
};
static minf_status ragged_layout(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* seq_lens,
                                 RaggedLayout* L) {
  g_err[0] = 0;
  if (!prob || !heads) return fail(MINF_EINVAL, "null problem or head table");
  if (!seq_lens) return fail(MINF_EINVAL, "null seq_lens");
  if (prob->B < 1) return fail(MINF_EINVAL, "B must be >= 1 (B=%d)", prob->B);
  int n_max = 0;
  for (int b = 0; b < prob->B; ++b) {
    if (seq_lens[b] < 1 || seq_lens[b] > prob->n)
      return fail(MINF_EINVAL, "sequence %d has length %d, outside [1, n=%d]", b, seq_lens[b], prob->n);
    n_max = std::max(n_max, seq_lens[b]);
  }
  Carve c;
  size_t stage = 256;
  L->r.assign((size_t)prob->B, RaggedRegion{});
  const size_t Hq = (size_t)prob->Hq;
  for (int b = 0; b < prob->B; ++b) {
    minf_problem one = *prob;
    one.B = 1;
    one.n = seq_lens[b];
    RaggedRegion& R = L->r[(size_t)b];
    minf_status s = validate(&one, heads, &R.d);
    if (s != MINF_OK) return s;
    const Derived& d = R.d;
    const size_t nq = (size_t)d.nq;
    R.vert = c.take(4 * Hq * std::max<int64_t>(d.max_v, 1));
    R.slash = c.take(4 * Hq * std::max<int64_t>(d.max_s, 1));
    R.blk = c.take(4 * Hq * nq * std::max<int64_t>(d.max_kb, 1));
    R.blkcnt = c.take(4 * Hq * nq);
    R.span_lo = c.take(4 * Hq * std::max<int64_t>(d.max_s, 1));
    R.span_hi = c.take(4 * Hq * std::max<int64_t>(d.max_s, 1));
    R.span_cnt = c.take(4 * Hq);
    R.chunk_lo = c.take(4 * Hq * std::max<int64_t>(d.max_chunks, 1));
    R.chunk_hi = c.take(4 * Hq * std::max<int64_t>(d.max_chunks, 1));
    R.chunk_cnt = c.take(4 * Hq * nq);
    R.cols = c.take(4 * Hq * nq * std::max<int64_t>(d.max_v, 1));
    R.col_cnt = c.take(4 * Hq * nq);
    R.sbits = c.take(4 * Hq * std::max<int64_t>(d.bits_words, 1));
    R.cbits = c.take(4 * Hq * std::max<int64_t>(d.bits_words, 1));
    R.tail_x = c.take(4 * Hq * std::max<int64_t>(d.max_tail, 1));
    R.tail_cnt = c.take(4 * Hq);
    R.pk_cnt = c.take(4 * Hq * nq);
    stage = std::max(stage, ws_total(&one, d));
  }
  L->all = *prob;
  L->all.n = n_max;
  minf_status s = validate(&L->all, heads, &L->d_all);
  if (s != MINF_OK) return s;
  L->stage_bytes = stage;
  L->stage = c.take(stage);
  L->attn = c.take(attn_ws(&L->all, L->d_all).total);
  L->table = c.take(sizeof(minf::SampleDesc) * (size_t)prob->B);
  L->kept = c.take(8 * Hq);
  L->total = c.off;
  return MINF_OK;
}

minf_status minf_output_error(const minf_problem* prob, const void* O, const void* O_ref, double* err, void* stream) {
  g_err[0] = 0;
  if (!prob || !O || !O_ref || !err) return fail(MINF_EINVAL, "null problem, O, O_ref or err");
  if (prob->B < 1 || prob->n < 1 || prob->Hq < 1 || prob->Hq > MINF_MAX_HEADS)
    return fail(MINF_EINVAL, "B, n must be >= 1 and Hq in [1, %d] (B=%d n=%d Hq=%d)", MINF_MAX_HEADS, prob->B, prob->n,
                prob->Hq);
  if (prob->dh != 64 && prob->dh != 128) return fail(MINF_EUNSUPPORTED, "dh must be 64 or 128 (dh=%d)", prob->dh);
  if (prob->out_dtype != MINF_F32 && prob->out_dtype != MINF_BF16)
    return fail(MINF_EINVAL, "bad out_dtype %d", prob->out_dtype);
  return hip_status(minf::launch_output_error(O, O_ref, (int64_t)prob->B * prob->Hq, (int64_t)prob->n * prob->dh,
                                              prob->out_dtype == MINF_BF16, err, static_cast<hipStream_t>(stream)),
                    "minf_output_error launch");
}

minf_status minf_captured_mass(const minf_problem* prob, const float* lse, const float* lse_ref, double* mass,
                               void* stream) {
  g_err[0] = 0;
  if (!prob || !lse || !lse_ref || !mass) return fail(MINF_EINVAL, "null problem, lse, lse_ref or mass");
  if (prob->B < 1 || prob->n < 1 || prob->Hq < 1 || prob->Hq > MINF_MAX_HEADS)
    return fail(MINF_EINVAL, "B, n must be >= 1 and Hq in [1, %d] (B=%d n=%d Hq=%d)", MINF_MAX_HEADS, prob->B, prob->n,
                prob->Hq);
  return hip_status(minf::launch_captured_mass(lse, lse_ref, (int64_t)prob->B * prob->Hq, prob->n, mass,
                                               static_cast<hipStream_t>(stream)),
                    "minf_captured_mass launch");
}

minf_status minf_ragged_ws_bytes(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* seq_lens,
                                 int64_t* ws_bytes) {
  g_err[0] = 0;
  if (!ws_bytes) return fail(MINF_EINVAL, "null ws_bytes");
  RaggedLayout L;
  const minf_status s = ragged_layout(prob, heads, seq_lens, &L);
  if (s != MINF_OK) return s;
  *ws_bytes = (int64_t)L.total;
  return MINF_OK;
}

minf_status minf_prefill_ragged(const minf_problem* prob, const minf_head_cfg* heads, const int32_t* seq_lens,
                                const void* Q, const void* K, const void* V, void* O, float* lse,
                                int64_t* kept_edges, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  RaggedLayout L;
  minf_status s = ragged_layout(prob, heads, seq_lens, &L);
  if (s != MINF_OK) return s;
  if (!Q || !K || !V || !O || !status) return fail(MINF_EINVAL, "null Q, K, V, O or status");
  if (!ws) return fail(MINF_EWORKSPACE, "workspace pointer is null");
  if (ws_bytes < L.total) return fail(MINF_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                                      L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = hip_status(minf::launch_fill_i32(status, 1, 0, st), "status reset")) != MINF_OK) return s;
  char* w = static_cast<char*>(ws);
  const size_t in_sz = prob->in_dtype == MINF_BF16 ? 2 : 4;
  const size_t Hq = (size_t)prob->Hq, Hkv = (size_t)prob->Hkv, dh = (size_t)prob->dh;
  minf::SampleDesc* table = reinterpret_cast<minf::SampleDesc*>(w + L.table);
  minf::SampleBatch batch{};
  int in_batch = 0;
  size_t off = 0;   // tokens before sample b
  // index and tile stages, one sequence after another (each a B = 1
  // problem of its own length, into its own region); the descriptors of the
  // sequences go to the table in batches
  for (int b = 0; b < prob->B; ++b) {
    const RaggedRegion& R = L.r[(size_t)b];
    minf_problem one = *prob;
    one.B = 1;
    one.n = seq_lens[b];
    minf_tiles t{};
    t.span_lo = reinterpret_cast<int32_t*>(w + R.span_lo);
    t.span_hi = reinterpret_cast<int32_t*>(w + R.span_hi);
    t.span_cnt = reinterpret_cast<int32_t*>(w + R.span_cnt);
    t.chunk_lo = reinterpret_cast<int32_t*>(w + R.chunk_lo);
    t.chunk_hi = reinterpret_cast<int32_t*>(w + R.chunk_hi);
    t.chunk_cnt = reinterpret_cast<int32_t*>(w + R.chunk_cnt);
    t.cols = reinterpret_cast<int32_t*>(w + R.cols);
    t.col_cnt = reinterpret_cast<int32_t*>(w + R.col_cnt);
    t.slash_bits = reinterpret_cast<uint32_t*>(w + R.sbits);
    t.col_bits = reinterpret_cast<uint32_t*>(w + R.cbits);
    t.tail_x = reinterpret_cast<int32_t*>(w + R.tail_x);
    t.tail_cnt = reinterpret_cast<int32_t*>(w + R.tail_cnt);
    t.pk_cnt = reinterpret_cast<int32_t*>(w + R.pk_cnt);
    t.status = status;
    // kept edges of this sample go straight to the caller's [B, Hq] array,
    // or to a scratch row of the workspace
    t.kept_edges = kept_edges ? kept_edges + (size_t)b * Hq : reinterpret_cast<int64_t*>(w + L.kept);
    int32_t* vert = reinterpret_cast<int32_t*>(w + R.vert);
    int32_t* slash = reinterpret_cast<int32_t*>(w + R.slash);
    int32_t* blk = reinterpret_cast<int32_t*>(w + R.blk);
    int32_t* blkcnt = reinterpret_cast<int32_t*>(w + R.blkcnt);
    void* stage = w + L.stage;
    const char* Qb = static_cast<const char*>(Q) + in_sz * Hq * dh * off;
    const char* Kb = static_cast<const char*>(K) + in_sz * Hkv * dh * off;
    if ((s = minf_vs_index(&one, heads, Qb, Kb, vert, slash, nullptr, nullptr, stage, L.stage_bytes, stream)) != MINF_OK ||
        (s = minf_bs_index(&one, heads, Qb, Kb, blk, blkcnt, stage, L.stage_bytes, stream)) != MINF_OK ||
        (s = minf_build_tiles(&one, heads, vert, slash, blk, blkcnt, &t, stage, L.stage_bytes, stream)) != MINF_OK)
      return s;
    minf::SampleDesc& D = batch.d[in_batch++];
    D = minf::SampleDesc{};
    D.q_row = (int64_t)(Hq * off);
    D.kv_row = (int64_t)(Hkv * off);
    D.chunk_lo = t.chunk_lo; D.chunk_hi = t.chunk_hi; D.chunk_cnt = t.chunk_cnt;
    D.cols = t.cols; D.col_cnt = t.col_cnt;
    D.blk_idx = blk; D.blk_cnt = blkcnt;
    D.slash_bits = R.d.bits_words > 0 ? t.slash_bits : nullptr;
    D.col_bits = R.d.bits_words > 0 ? t.col_bits : nullptr;
    D.tail_x = t.tail_x; D.pk_cnt = t.pk_cnt;
    D.max_chunks = R.d.max_chunks; D.max_v = R.d.max_v; D.max_kb = R.d.max_kb; D.bits_words = R.d.bits_words;
    D.max_tail = R.d.max_tail;
    D.n = seq_lens[b];
    D.nq = (int32_t)R.d.nq;
    if (in_batch == minf::kSampleBatch || b + 1 == prob->B) {
      batch.dst = table + (b + 1 - in_batch);
      batch.count = in_batch;
      if ((s = hip_status(minf::launch_write_samples(batch, st), "sequence table")) != MINF_OK) return s;
      in_batch = 0;
    }
    off += (size_t)seq_lens[b];
  }
  // the attention of every sequence in one launch
  minf_tiles none{};
  return attn_launch(&L.all, L.d_all, Q, K, V, nullptr, nullptr, &none, O, lse, w + L.attn, stream,
                     "minf_prefill_ragged attention launch", table);
}

minf_status minf_timing_start(int32_t max_calls) {
  if (max_calls < 1 || max_calls > 65536) return fail(MINF_EINVAL, "max_calls %d outside [1, 65536]", max_calls);
  timing_release();
  std::vector<hipEvent_t> ev(2 * (size_t)max_calls, nullptr);
  for (size_t i = 0; i < ev.size(); ++i) {
    const hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return hip_status(e, "minf_timing_start: hipEventCreate");
    }
  }
  g_timing.ev = std::move(ev);
  g_timing.cap = max_calls;
  return MINF_OK;
}

minf_status minf_timing_read(float* ms, int32_t cap, int32_t* count) {
  if (!count || (cap > 0 && !ms) || cap < 0) return fail(MINF_EINVAL, "null count or output array");
  if (g_timing.cap == 0) return fail(MINF_EINVAL, "minf_timing_start was not called");
  minf_status s = hip_status(g_timing.err, "minf_timing: hipEventRecord");
  const int used = g_timing.used;
  for (int i = 0; s == MINF_OK && i < used && i < cap; ++i) {
    s = hip_status(hipEventSynchronize(g_timing.ev[2 * i + 1]), "minf_timing_read: hipEventSynchronize");
    if (s == MINF_OK)
      s = hip_status(hipEventElapsedTime(&ms[i], g_timing.ev[2 * i], g_timing.ev[2 * i + 1]),
                     "minf_timing_read: hipEventElapsedTime");
  }
  *count = used;
  timing_release();
  return s;
}

}  // extern "C"
