"""CPU fp64 oracle for MInference-style dynamic-sparse causal attention prefill.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never touches it and
shares no code with it.

Everything here is a plain, slow, step-by-step restatement of what the pages
define, in float64 NumPy; the restricted softmax over explicit key ranges for
long sequences is plain C in double precision (oracle/attend.c, compiled by
build_c()).  Sources (cited by page title and section):

* [MInf]  PaperTrace 2.1.2 "MInference: 按 head 模式加速长上下文 Prefill"
* [Blog]  blog-zz7 "LLM模型之MInference", section 2.3
* [Cost]  PaperTrace 1.1.1 "成本模型：训练、prefill、解码与 KV cache"

Readings taken where the pages are open:

* slash expansion: a slash offset d covers, for the query block u of
  ``slash_tile`` rows, the keys [t*u - d, t*u + t - 1 - d]  (t = slash_tile;
  t = 64 is the physical 64x64 tile of [MInf] section 2.1; t = 1 is Eq. 5);
* vertical columns are exact single keys ([MInf] section 4.1);
* the VS proxy statistic is the causal softmax probability summed over the
  last ``last_q`` rows, with no length normalisation ([MInf] section 6.2);
* the BS proxy is mean pooling + scaled dot product, no softmax
  ([MInf] section 2, Block-Sparse; [Blog] section 2.3.2);
* top-k orders by (score descending, index ascending) and returns the chosen
  indices sorted ascending;
* an empty candidate row gives o = 0 and LSE = -inf;
* the pattern search ([MInf] sections 3.1 and 6.3; [Blog] section 2.3.1)
  measures a candidate by its missed attention mass 1 - m (m the row mean of
  the dense softmax mass its kept keys carry; Eq. 2's L1 row distance is
  2 (1 - m)) or by its relative output error, and keeps per head the least
  time among candidates within the bound, ties to the earlier candidate.

Parity status: every function below is pinned by tests/test_oracle_*.py
against values printed on the pages, closed forms, invariants, special cases
that reduce to library routines, or the loop-only brute force in brute.py.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, List, Optional, Sequence

import numpy as np

ASHAPE, VSLASH, BSPARSE = 0, 1, 2
FORCE_FIRST_BLOCK, FORCE_DIAG_BLOCK = 1, 2
BLOCK = 64


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of what the GPU reads: bf16 bit patterns are
    widened by placing them in the high half of a float32."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """GQA map: query head h reads KV head floor(h / (Hq/Hkv))
    ([MInf] section 5.1, "head 分派与 GQA 映射")."""
    return h // (Hq // Hkv)


def n_blocks(n: int, block: int = BLOCK) -> int:
    return (n + block - 1) // block


# ----------------------------------------------------------------------------
# dense causal attention: [MInf] section 1.1, Eq. 1-2
# ----------------------------------------------------------------------------

def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """o_i = sum_{j<=i} softmax_j(scale * q_i.k_j) v_j for every row, one head."""
    n = q.shape[0]
    s = scale * (q @ k.T)
    s[np.triu_indices(n, 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, (m + np.log(l))[:, 0]


# ----------------------------------------------------------------------------
# top-k selection: ties go to the lowest index
# ----------------------------------------------------------------------------

def topk_ascending(scores: np.ndarray, k: int, index: Optional[np.ndarray] = None) -> np.ndarray:
    """The first min(k, len) candidates under (score descending, index
    ascending), returned sorted ascending by index."""
    scores = np.asarray(scores, dtype=np.float64)
    if index is None:
        index = np.arange(scores.shape[0], dtype=np.int64)
    k = min(int(k), scores.shape[0])
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((index, -scores))          # last key is primary
    return np.sort(index[order[:k]])


def kth_threshold(scores: np.ndarray, k: int) -> float:
    """Score of the k-th selected candidate (the selection threshold t_k)."""
    k = min(int(k), scores.shape[0])
    if k <= 0:
        return math.inf
    return float(np.sort(np.asarray(scores, dtype=np.float64))[::-1][k - 1])


# ----------------------------------------------------------------------------
# Vertical-Slash index: [MInf] section 6.2 (proxy), section 2.1 (Eq. 5);
# [Blog] section 2.3.2 (last_q rows against all keys)
# ----------------------------------------------------------------------------

def vs_proxy_scores(q: np.ndarray, k: np.ndarray, last_q: int, scale: float):
    """Column scores c_j and diagonal scores r_d of one query head.

    The sampled rows are the last min(last_q, n) queries.  For each sampled
    row i the proxy weights are the causal softmax over keys j <= i of
    scale*q_i.k_j; c_j sums them over the sampled rows, r_d sums the weight
    of the pair (i, i-d) over the sampled rows.
    """
    n = q.shape[0]
    L = min(int(last_q), n)
    rows = np.arange(n - L, n)
    s = scale * (q[rows] @ k.T)                    # [L, n]
    s[rows[:, None] < np.arange(n)[None, :]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    a = e / e.sum(axis=1, keepdims=True)           # proxy softmax, rows sum to 1
    c = a.sum(axis=0)
    r = np.zeros(n)
    for t, i in enumerate(rows):                   # weight of (i, i-d) goes to r_d
        r[: i + 1] += a[t, i::-1]
    return c, r


def vs_index(q, k, last_q, n_vertical, n_slash, scale):
    """C_h = top-v columns of c, D_h = top-s offsets of r ([MInf] section 6.2)."""
    c, r = vs_proxy_scores(q, k, last_q, scale)
    return topk_ascending(c, n_vertical), topk_ascending(r, n_slash), c, r


# ----------------------------------------------------------------------------
# Block-Sparse index: [MInf] section 2 (Eq. 6, mean pooling); [Blog] 2.3.2
# ----------------------------------------------------------------------------

def block_means(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Mean of each run of `block` rows (the last block over its true length)."""
    n = x.shape[0]
    nb = n_blocks(n, block)
    out = np.empty((nb, x.shape[1]))
    for u in range(nb):
        out[u] = x[u * block:min(n, (u + 1) * block)].mean(axis=0)
    return out


def bs_block_scores(q, k, scale, block: int = BLOCK) -> np.ndarray:
    """r_uv = scale * mean(Q block u) . mean(K block v) for v <= u; -inf above."""
    qb, kb = block_means(q, block), block_means(k, block)
    r = scale * (qb @ kb.T)
    nb = r.shape[0]
    r[np.triu_indices(nb, 1)] = -np.inf
    return r


def bs_index(q, k, topk, force_flags, scale, block: int = BLOCK) -> List[np.ndarray]:
    """J_u = TopK_{v<=u}(r_uv, k_b), sorted ascending (Eq. 6).  Forced blocks
    (first and/or diagonal) take score +inf and so occupy budget slots."""
    r = bs_block_scores(q, k, scale, block)
    nb = r.shape[0]
    out = []
    for u in range(nb):
        row = r[u, :u + 1].copy()
        if force_flags & FORCE_FIRST_BLOCK:
            row[0] = np.inf
        if force_flags & FORCE_DIAG_BLOCK:
            row[u] = np.inf
        out.append(topk_ascending(row, topk))
    return out


# ----------------------------------------------------------------------------
# candidate sets N_h(i)
# ----------------------------------------------------------------------------

def ashape_mask(rows: np.ndarray, nkeys: int, sink: int, window: int) -> np.ndarray:
    """Eq. 3: j in [0, min(g-1, i)] or j in [max(0, i-w+1), i]."""
    i = rows[:, None]
    j = np.arange(nkeys)[None, :]
    return (j <= i) & ((j < sink) | (j >= i - window + 1))


def slash_offset_set(offs: np.ndarray, n: int, slash_tile: int) -> np.ndarray:
    """Boolean over x in [-(t-1), n): x is in the union of [d-t+1, d] for
    d in D.  Key j of query block u is slash-covered iff t*u - j is in it."""
    t = slash_tile
    cover = np.zeros(n + t - 1, dtype=bool)        # index x + t - 1
    for d in np.asarray(offs, dtype=np.int64):
        cover[d: d + t] = True                     # x in [d-t+1, d]
    return cover


def vs_mask(rows: np.ndarray, nkeys: int, n: int, cols, offs, slash_tile: int,
            cover: Optional[np.ndarray] = None) -> np.ndarray:
    """Eq. 5 with the slash expansion reading: j <= i and (j in C_h or j is
    covered by a slash of D_h expanded to the t x t tile of row i's block).

    Key j of block u is covered iff x = t*u - j lies in the union of
    [d-t+1, d] over d in D_h (see slash_offset_set).
    """
    t = slash_tile
    if cover is None:
        cover = slash_offset_set(offs, n, t)
    rows = np.asarray(rows, dtype=np.int64)
    i = rows[:, None]
    j = np.arange(nkeys)[None, :]
    # Key j of row i's block u is covered iff cover[t*u - j + t - 1] (the
    # offset x = t*u - j, stored at x + t - 1).  Read along j, that is the
    # array `cover` backwards from position t*u + t - 1; with `rev` the
    # reversed array (followed by zeros for x < -(t-1), i.e. keys past the
    # block), cover[t*u + t - 1 - j] = rev[L - t - t*u + j], L = len(cover).
    L = cover.shape[0]
    rev = np.zeros(L + nkeys, dtype=bool)
    rev[:L] = cover[::-1]
    start = L - t - t * (rows // t)               # >= 0: t*u <= i <= n - 1 = L - t
    covered = np.lib.stride_tricks.sliding_window_view(rev, nkeys)[start]
    colset = np.zeros(nkeys, dtype=bool)
    cc = np.asarray(cols, dtype=np.int64)
    colset[cc[cc < nkeys]] = True
    return (j <= i) & (covered | colset[None, :])


def bs_mask(rows: np.ndarray, nkeys: int, J: Sequence[np.ndarray], block: int = BLOCK) -> np.ndarray:
    """Eq. 6: j <= i and block(j) in J_{block(i)}."""
    nb = len(J)
    sel = np.zeros((nb, n_blocks(nkeys, block)), dtype=bool)
    for u, jj in enumerate(J):
        jj = np.asarray(jj, dtype=np.int64)
        sel[u, jj[jj < sel.shape[1]]] = True
    i = rows[:, None]
    j = np.arange(nkeys)[None, :]
    return (j <= i) & sel[rows // block][:, np.arange(nkeys) // block]


# ----------------------------------------------------------------------------
# restricted softmax: [MInf] section 1.1 (Eq. 2 over N_h(i)), section 3.2
# ----------------------------------------------------------------------------

def attend_rows(q, k, v, rows: np.ndarray, mask_fn: Callable, scale: float, chunk: int = 64):
    """o_i and LSE_i for the given rows, summing only over N_h(i).

    Rows are handled in chunks: the scores against keys [0, max row] are a
    dense product, excluded pairs are removed before the row maximum (they
    never enter the max or the sum), and the softmax is taken in float64.
    An empty row gives o = 0 and LSE = -inf.
    """
    rows = np.asarray(rows, dtype=np.int64)
    dh = v.shape[1]
    o = np.zeros((rows.shape[0], dh))
    lse = np.full(rows.shape[0], -np.inf)
    order = np.argsort(rows, kind="stable")
    for s in range(0, rows.shape[0], chunk):
        idx = order[s:s + chunk]
        rr = rows[idx]
        nk = int(rr.max()) + 1
        mask = mask_fn(rr, nk)
        sc = scale * (q[rr] @ k[:nk].T)
        sc[~mask] = -np.inf
        m = sc.max(axis=1)
        ok = np.isfinite(m)
        mm = np.where(ok, m, 0.0)
        p = np.exp(sc - mm[:, None])              # exp(-inf) = 0 for excluded pairs
        l = p.sum(axis=1)
        num = p @ v[:nk]
        o[idx[ok]] = num[ok] / l[ok, None]
        lse[idx[ok]] = mm[ok] + np.log(l[ok])
    return o, lse


# ----------------------------------------------------------------------------
# one row at a time: the candidate keys of row i listed explicitly, and the
# restricted softmax over them.  For long sequences, where a dense mask of
# many rows against all keys does not fit; same definitions as above.
# ----------------------------------------------------------------------------

def ashape_row_keys(i: int, sink: int, window: int) -> np.ndarray:
    """N(i) of Eq. 3, ascending: [0, min(g-1, i)] united with [max(0, i-w+1), i]."""
    j = np.arange(i + 1, dtype=np.int64)
    return j[(j < sink) | (j >= i - window + 1)]


def vs_row_keys(i: int, cols, cover: np.ndarray, slash_tile: int) -> np.ndarray:
    """N(i) of the VS set, ascending: keys j <= i of row i's query block
    u = i // t that a slash covers (t*u - j in S, `cover` from
    slash_offset_set), united with the columns j <= i."""
    t = slash_tile
    u = i // t
    x = np.nonzero(cover)[0] - (t - 1)             # the covered offsets x
    j = t * u - x
    j = j[(j >= 0) & (j <= i)]
    c = np.asarray(cols, dtype=np.int64)
    c = c[c <= i]
    return np.union1d(j, c)


def bs_row_keys(i: int, J: Sequence[np.ndarray], block: int = BLOCK) -> np.ndarray:
    """N(i) of Eq. 6, ascending: keys j <= i whose block is in J_{i // block}."""
    out = []
    for v in np.sort(np.asarray(J[i // block], dtype=np.int64)):
        lo = v * block
        hi = min(lo + block - 1, i)
        if lo <= hi:
            out.append(np.arange(lo, hi + 1, dtype=np.int64))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def attend_row_keys(q_i: np.ndarray, k: np.ndarray, v: np.ndarray, keys: np.ndarray, scale: float):
    """o_i and LSE_i of Eq. 2 over the listed keys: the softmax of
    scale * q_i . k_j over j in keys, applied to v_j (o = 0, LSE = -inf when
    the list is empty)."""
    if keys.shape[0] == 0:
        return np.zeros(v.shape[1]), -np.inf
    s = scale * (k[keys] @ q_i)
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ v[keys]) / l, m + math.log(l)


# ----------------------------------------------------------------------------
# row by row over key ranges, in C (oracle/attend.c): the same restricted
# softmax for long sequences, where a row keeps few of the keys before it.
# N(i) is listed as disjoint inclusive key ranges; the ranges below are the
# sets of Eq. 3, of the slash expansion / Eq. 5 and of Eq. 6.
# ----------------------------------------------------------------------------

_CLIB = None
_C_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attend.c")
_C_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboracle.so")


def build_c(force: bool = False) -> str:
    """Compile oracle/attend.c into oracle/liboracle.so with the host C
    compiler (plain -O2, IEEE arithmetic)."""
    import subprocess
    if force or not os.path.exists(_C_LIB) or os.path.getmtime(_C_LIB) < os.path.getmtime(_C_SRC):
        tmp = _C_LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", _C_SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _C_LIB)
    return _C_LIB


def _clib():
    global _CLIB
    if _CLIB is None:
        import ctypes
        lib = ctypes.CDLL(build_c())
        f = lib.oracle_attend_ranges
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int64, ctypes.c_int64, P, P, P, P, P, P, ctypes.c_double, P, P]
        f.restype = ctypes.c_int
        _CLIB = lib
    return _CLIB


def ashape_row_ranges(i: int, sink: int, window: int):
    """N(i) of Eq. 3 as disjoint ranges: the sinks [0, min(g-1, i)] and the
    part of the window [max(0, i-w+1), i] that lies past them."""
    lo, hi = [], []
    a = min(sink - 1, i)
    if a >= 0:
        lo.append(0)
        hi.append(a)
    b = max(sink, i - window + 1, 0)
    if window > 0 and b <= i:
        lo.append(b)
        hi.append(i)
    return np.array(lo, dtype=np.int64), np.array(hi, dtype=np.int64)


def bs_row_ranges(i: int, J: Sequence[np.ndarray], block: int = BLOCK):
    """N(i) of Eq. 6 as ranges: each selected block of row i's query block,
    cut at the row (causal)."""
    v = np.sort(np.asarray(J[i // block], dtype=np.int64))
    lo = v * block
    hi = np.minimum(lo + block - 1, i)
    keep = lo <= hi
    return lo[keep], hi[keep]


def span_runs(cover: np.ndarray, slash_tile: int):
    """The covered offsets x (cover from slash_offset_set, indexed x + t - 1)
    as sorted disjoint inclusive runs [a, b]."""
    d = np.diff(np.concatenate([[0], cover.astype(np.int8), [0]]))
    a = np.flatnonzero(d == 1)
    b = np.flatnonzero(d == -1) - 1
    return a - (slash_tile - 1), b - (slash_tile - 1)


def vs_row_ranges(i: int, cols, cover: np.ndarray, slash_tile: int, runs=None):
    """N(i) of the VS set as disjoint ranges: for row i's query block
    u = i // t, the keys j = t*u - x of every covered run of offsets x,
    clipped to [0, i], then each column j <= i that no slash of block u
    covers, as a range of one key."""
    t = slash_tile
    xa, xb = span_runs(cover, t) if runs is None else runs
    u = i // t
    lo = np.maximum(t * u - xb, 0)
    hi = np.minimum(t * u - xa, i)
    keep = lo <= hi
    c = np.asarray(cols, dtype=np.int64)
    c = c[c <= i]
    unc = c[~cover[t * u - c + t - 1]]
    return np.concatenate([lo[keep], unc]), np.concatenate([hi[keep], unc])


def attend_rows_ranges(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                       ranges_fn: Callable, scale: float):
    """o_i and LSE_i for the given rows over N(i) = ranges_fn(i) (disjoint
    inclusive key ranges), in double precision (attend.c).  q_rows [R, dh]
    are rows `rows` of Q; k, v [n, dh]; all float32 values (bf16 widens to
    float32 exactly).  Empty rows give o = 0 and LSE = -inf."""
    rows = np.asarray(rows, dtype=np.int64)
    R, dh = rows.shape[0], k.shape[1]
    los, his, ptr = [], [], [0]
    for i in rows:
        lo, hi = ranges_fn(int(i))
        los.append(lo)
        his.append(hi)
        ptr.append(ptr[-1] + lo.shape[0])
    lo = np.ascontiguousarray(np.concatenate(los) if los else np.zeros(0), dtype=np.int64)
    hi = np.ascontiguousarray(np.concatenate(his) if his else np.zeros(0), dtype=np.int64)
    ptr = np.asarray(ptr, dtype=np.int64)
    assert np.all(lo >= 0) and np.all(hi < k.shape[0]) and np.all(hi <= np.repeat(rows, np.diff(ptr)))
    q = np.ascontiguousarray(q_rows, dtype=np.float32)
    kk = np.ascontiguousarray(k, dtype=np.float32)
    vv = np.ascontiguousarray(v, dtype=np.float32)
    o = np.zeros((R, dh))
    lse = np.zeros(R)
    rc = _clib().oracle_attend_ranges(R, dh, q.ctypes.data, kk.ctypes.data, vv.ctypes.data, ptr.ctypes.data,
                                      lo.ctypes.data, hi.ctypes.data, float(scale), o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_attend_ranges: out of memory")
    return o, lse


# ----------------------------------------------------------------------------
# kept edges E_h = sum_i |N_h(i)|  ([MInf] section 1.2)
# ----------------------------------------------------------------------------

def ashape_row_counts(n: int, sink: int, window: int) -> np.ndarray:
    """|N(i)| for Eq. 3, by interval arithmetic on the two sets."""
    i = np.arange(n, dtype=np.int64)
    a_hi = np.minimum(sink - 1, i)                 # sinks [0, a_hi]
    b_lo = np.maximum(0, i - window + 1)           # window [b_lo, i]
    na = np.maximum(0, a_hi + 1)
    nb = np.maximum(0, i - b_lo + 1)
    ov = np.maximum(0, np.minimum(a_hi, i) - b_lo + 1)
    return na + nb - ov


def vs_row_counts(n: int, cols, offs, slash_tile: int) -> np.ndarray:
    """|N(i)| for the VS set: slash-covered keys in [0, i] plus the columns
    <= i that no slash covers."""
    t = slash_tile
    cover = slash_offset_set(offs, n, t)           # index x + t - 1
    pref = np.concatenate([[0], np.cumsum(cover)])  # pref[a] = #{covered x < a - t + 1}
    i = np.arange(n, dtype=np.int64)
    u = i // t
    r = i - t * u
    # keys j = t*u - x in [0, i]  <=>  x in [-r, t*u]
    span = pref[t * u + t] - pref[-r + t - 1]
    cc = np.sort(np.asarray(cols, dtype=np.int64))
    colcnt = np.zeros(n, dtype=np.int64)
    for uu in range(n_blocks(n, t)):
        r0, r1 = t * uu, min(n, t * uu + t)
        c = cc[cc < r1]
        x = t * uu - c
        unc = c[~cover[x + t - 1]]
        colcnt[r0:r1] = np.searchsorted(unc, np.arange(r0, r1), side="right")
    return span + colcnt


def vs_edges(n: int, cols, offs, slash_tile: int) -> int:
    """sum_i |N(i)| for the VS set, without materialising per-row counts of
    the columns: a column c adds, in block u, the rows of u at or after c,
    unless a slash covers it there."""
    t = slash_tile
    cover = slash_offset_set(offs, n, t)
    pref = np.concatenate([[0], np.cumsum(cover)])
    i = np.arange(n, dtype=np.int64)
    u = i // t
    r = i - t * u
    span = int((pref[t * u + t] - pref[-r + t - 1]).sum())
    cc = np.sort(np.asarray(cols, dtype=np.int64))
    cc = cc[cc < n]
    if t == 1:
        # row i keeps column c (c <= i) unless i - c is a slash offset
        d = np.sort(np.asarray(offs, dtype=np.int64))
        hit = np.searchsorted(d, n - 1 - cc, side="right")
        return span + int(((n - cc) - hit).sum())
    nb = n_blocks(n, t)
    tot = 0
    for uu in range(nb):
        r0, r1 = t * uu, min(n, t * uu + t)
        c = cc[cc < r1]
        unc = c[~cover[t * uu - c + t - 1]]
        tot += int((r1 - np.maximum(unc, r0)).sum())
    return span + tot


def bs_edges(n: int, J: Sequence[np.ndarray], block: int = BLOCK) -> int:
    tot = 0
    for u, jj in enumerate(J):
        lu = min(block, n - u * block)
        for v in np.asarray(jj, dtype=np.int64):
            if v < u:
                tot += lu * min(block, n - v * block)
            elif v == u:
                tot += lu * (lu + 1) // 2
    return int(tot)


# ----------------------------------------------------------------------------
# one layer
# ----------------------------------------------------------------------------

class HeadResult:
    __slots__ = ("kind", "cols", "offs", "c", "r", "J", "edges", "edges_eq5", "mask_fn")


def _cfg(c):
    """Accept either a HeadCfg-like object or a tuple in minf_head_cfg order."""
    if hasattr(c, "as_tuple"):
        c = c.as_tuple()
    kind, sink, window, last_q, nv, ns, kb, ff = (int(x) for x in c)
    return kind, sink, window, last_q, nv, ns, kb, ff


def head_index(q, k, cfg, n: int, scale: float, slash_tile: int = 64, block: int = BLOCK,
               given=None) -> HeadResult:
    """Index estimation + candidate set of one (batch, head).

    `given` may supply (cols, offs) for a VS head or J for a BS head instead
    of estimating them from Q and K.
    """
    kind, sink, window, last_q, nv, ns, kb, ff = _cfg(cfg)
    res = HeadResult()
    res.kind = kind
    res.cols = res.offs = res.c = res.r = res.J = None
    if kind == ASHAPE:
        res.edges = int(ashape_row_counts(n, sink, window).sum())
        res.edges_eq5 = res.edges
        res.mask_fn = lambda rows, nk: ashape_mask(rows, nk, sink, window)
    elif kind == VSLASH:
        if given is None:
            res.cols, res.offs, res.c, res.r = vs_index(q, k, last_q, nv, ns, scale)
        else:
            res.cols, res.offs = (np.asarray(x, dtype=np.int64) for x in given)
        cols, offs = res.cols, res.offs
        res.edges = vs_edges(n, cols, offs, slash_tile)
        res.edges_eq5 = vs_edges(n, cols, offs, 1)
        cover = slash_offset_set(offs, n, slash_tile)
        res.mask_fn = lambda rows, nk: vs_mask(rows, nk, n, cols, offs, slash_tile, cover)
    elif kind == BSPARSE:
        if given is None:
            res.J = bs_index(q, k, kb, ff, scale, block)
        else:
            res.J = [np.asarray(x, dtype=np.int64) for x in given]
        J = res.J
        res.edges = bs_edges(n, J, block)
        res.edges_eq5 = res.edges
        res.mask_fn = lambda rows, nk: bs_mask(rows, nk, J, block)
    else:
        raise ValueError(f"unknown pattern kind {kind}")
    return res


def _workers(workers):
    if workers:
        return workers
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:
        c = os.cpu_count() or 1
    return max(1, min(16, c))


def run_layer(Q, K, V, dtype: str, heads, scale: float = 0.0, rows=None, slash_tile: int = 64,
              given=None, workers=None, attend: bool = True):
    """Whole-layer oracle: index (or given indices), kept edges and, on the
    requested rows (all rows if None), the restricted-softmax output.

    Q: [B, Hq, n, dh], K/V: [B, Hkv, n, dh] as float32 or bf16 bits.
    given: optional dict {(b, h): indices} overriding estimation.
    Returns a dict keyed by (b, h) of HeadResult, plus "O" [B, Hq, R, dh]
    and "LSE" [B, Hq, R] when attend is set.
    """
    B, Hq, n, dh = Q.shape
    Hkv = K.shape[1]
    sc = scale if scale else 1.0 / math.sqrt(dh)
    rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = {}
    O = np.zeros((B, Hq, rows.shape[0], dh)) if attend else None
    LSE = np.full((B, Hq, rows.shape[0]), -np.inf) if attend else None

    def one(bh):
        b, h = bh
        kv = kv_head(h, Hq, Hkv)
        q = widen(Q[b, h], dtype)
        k = widen(K[b, kv], dtype)
        g = None if given is None else given.get((b, h))
        res = head_index(q, k, heads[h], n, sc, slash_tile, BLOCK, g)
        if attend:
            v = widen(V[b, kv], dtype)
            O[b, h], LSE[b, h] = attend_rows(q, k, v, rows, res.mask_fn, sc)
        return bh, res

    items = [(b, h) for b in range(B) for h in range(Hq)]
    nw = _workers(workers)
    if nw > 1 and len(items) > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(nw) as ex:
            for bh, res in ex.map(one, items):
                out[bh] = res
    else:
        for bh in items:
            out[bh] = one(bh)[1]
    return {"heads": out, "O": O, "LSE": LSE, "rows": rows, "scale": sc}


# ----------------------------------------------------------------------------
# offline pattern search ([MInf] sections 3.1 and 6.3; [Blog] section 2.3.1,
# Eq. 2: each candidate's attention is compared with dense attention on a
# calibration input, and among acceptable candidates the faster is kept)
# ----------------------------------------------------------------------------

def output_error(O, O_ref):
    """Per head of [B, H, R, dh] outputs: (sum over batch, rows and columns of
    (O - O_ref)^2, sum of O_ref^2), both float64 arrays of length H."""
    a = np.asarray(O, dtype=np.float64)
    r = np.asarray(O_ref, dtype=np.float64)
    d = a - r
    return (d * d).sum(axis=(0, 2, 3)), (r * r).sum(axis=(0, 2, 3))


def relative_output_error(O, O_ref) -> np.ndarray:
    """||O_h - O_ref,h||_F / ||O_ref,h||_F per head (0 where both are 0)."""
    d2, r2 = output_error(O, O_ref)
    out = np.empty_like(d2)
    for h in range(d2.shape[0]):
        if r2[h] > 0:
            out[h] = math.sqrt(d2[h] / r2[h])
        else:
            out[h] = 0.0 if d2[h] == 0 else math.inf
    return out


def choose_patterns(err, times, eps: float) -> List[int]:
    """err [H, C] per-head errors of C candidates, times [C]: per head, the
    candidate of least time among those with error <= eps, ties to the
    lower candidate index; -1 where none qualifies."""
    err = np.asarray(err, dtype=np.float64)
    times = np.asarray(times, dtype=np.float64)
    out = []
    for h in range(err.shape[0]):
        ok = np.flatnonzero(err[h] <= eps)
        out.append(int(ok[np.argmin(times[ok])]) if ok.size else -1)
    return out


def captured_mass(q, k, rows: np.ndarray, mask_fn: Callable, scale: float, chunk: int = 64) -> np.ndarray:
    """Per row i of rows: the fraction of the dense causal softmax of row i
    (keys j <= i) that the keys kept by mask_fn carry ([MInf] section 3.1,
    the covered attention mass), from the explicit probabilities."""
    n = k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty(rows.shape[0])
    for s in range(0, rows.shape[0], chunk):
        r = rows[s:s + chunk]
        causal = np.arange(n)[None, :] <= r[:, None]
        sc = np.where(causal, scale * (q[r] @ k.T), -np.inf)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[s:s + r.shape[0]] = (p * (mask_fn(r, n) & causal)).sum(axis=1)
    return out


def layer_missed_mass(Q, K, dtype: str, heads, scale: float = 0.0, rows=None, workers=None) -> np.ndarray:
    """Per head h: 1 - the mean captured mass over the batch and the rows
    (all rows if None) under the layer's index estimation."""
    B, Hq, n, dh = Q.shape
    Hkv = K.shape[1]
    sc = scale if scale else 1.0 / math.sqrt(dh)
    rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    res = run_layer(Q, K, Q[:, :Hkv], dtype, heads, scale, rows=rows, attend=False, workers=workers)["heads"]
    out = np.zeros(Hq)
    for h in range(Hq):
        tot = 0.0
        for b in range(B):
            q = widen(Q[b, h], dtype)
            k = widen(K[b, kv_head(h, Hq, Hkv)], dtype)
            tot += captured_mass(q, k, rows, res[(b, h)].mask_fn, sc).sum()
        out[h] = 1.0 - tot / (B * rows.shape[0])
    return out
