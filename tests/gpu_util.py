"""Helpers shared by the GPU parity tests (not collected as tests).

Moves seeded problems to the device, feeds the oracle's index sets to the
GPU path, and compares results with the oracle element by element.
"""
import math
import sys
import time

import numpy as np

import long_context_prefill_amd as M
from oracle import minf_oracle as O

BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
F32_MAX_ABS, F32_MEAN_ABS = 1e-5, 1e-5
NEAR_TIE_REL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(p, device="cuda"):
    import torch
    if p.dtype == "bf16":
        conv = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device)
    else:
        conv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return conv(p.Q), conv(p.K), conv(p.V)


def make_prob(p, out_dtype="f32"):
    return M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, out_dtype, p.scale)


def load_oracle_indices(p, res, buf):
    """Write the oracle's VS / BS index sets into the GPU index buffers."""
    import torch
    sz = buf["sizes"]
    B, Hq, nq = p.B, p.Hq, int(sz.nq)
    vi = np.full((B, Hq, int(sz.max_v) or 1), -1, np.int32)
    si = np.full((B, Hq, int(sz.max_s)), -1, np.int32)
    bi = np.full((B, Hq, nq, int(sz.max_kb)), -1, np.int32)
    bc = np.zeros((B, Hq, nq), np.int32)
    for (b, h), r in res["heads"].items():
        if r.kind == O.VSLASH:
            vi[b, h, :len(r.cols)] = r.cols
            si[b, h, :len(r.offs)] = r.offs
        elif r.kind == O.BSPARSE:
            for u, J in enumerate(r.J):
                bi[b, h, u, :len(J)] = J
                bc[b, h, u] = len(J)
    dev = buf["vert_idx"].device
    buf["vert_idx"].copy_(torch.from_numpy(vi).to(dev))
    buf["slash_idx"].copy_(torch.from_numpy(si).to(dev))
    buf["blk_idx"].copy_(torch.from_numpy(bi).to(dev))
    buf["blk_cnt"].copy_(torch.from_numpy(bc).to(dev))


def gpu_given(p, buf, heads=None):
    """The GPU's own index sets in the form O.run_layer(given=...) takes:
    {(b, h): (cols, offs)} for Vertical-Slash heads and {(b, h): [J_u]} for
    Block-Sparse heads (the comparison protocol runs the oracle's attention
    on the GPU's index sets)."""
    vi = buf["vert_idx"].cpu().numpy()
    si = buf["slash_idx"].cpu().numpy()
    bi = buf["blk_idx"].cpu().numpy()
    bc = buf["blk_cnt"].cpu().numpy()
    out = {}
    for b in range(p.B):
        for h in (range(p.Hq) if heads is None else heads):
            kind = p.heads[h].kind
            if kind == O.VSLASH:
                out[(b, h)] = (vi[b, h][vi[b, h] >= 0].astype(np.int64), si[b, h][si[b, h] >= 0].astype(np.int64))
            elif kind == O.BSPARSE:
                out[(b, h)] = [bi[b, h, u, :bc[b, h, u]].astype(np.int64) for u in range(bi.shape[2])]
    return out


def check_block_selections(J, cnt, scores, k, force, what):
    """Every query block's Block-Sparse selection against the oracle's block
    scores at once, with the rule of check_selection: the GPU set of row u
    (J[u, :cnt[u]]) may differ from the oracle's top-min(k, u+1) set (score
    descending, index ascending) only in blocks whose oracle score lies within
    1e-4 relative of the row's threshold t_u, the k-th largest score.
    scores [nq, nq] fp64 (entries above the diagonal are ignored); forced
    blocks score +inf, so a row whose threshold is infinite must match
    exactly.  Returns (differing selections, exempt near-ties)."""
    nq = scores.shape[0]
    u = np.arange(nq)
    causal = np.arange(nq)[None, :] <= u[:, None]
    s = np.where(causal, np.asarray(scores, dtype=np.float64), -np.inf)
    if force & O.FORCE_FIRST_BLOCK:
        s[:, 0] = np.inf
    if force & O.FORCE_DIAG_BLOCK:
        s[u, u] = np.inf
    kk = np.minimum(int(k), u + 1)
    assert np.array_equal(np.asarray(cnt[:nq], dtype=np.int64), kk), f"{what}: block counts"
    width = J.shape[1]
    valid = np.arange(width)[None, :] < kk[:, None]
    Jv = np.where(valid, J[:nq, :width], 0).astype(np.int64)
    assert np.all((Jv >= 0) & (Jv <= u[:, None])), f"{what}: a block outside [0, u]"
    d = np.diff(np.where(valid, Jv, np.iinfo(np.int64).max), axis=1)
    assert np.all(d[valid[:, 1:]] > 0), f"{what}: blocks not strictly ascending"
    sel = np.zeros((nq, nq), dtype=bool)
    sel[np.repeat(u, width)[valid.ravel()], Jv[valid]] = True
    # t_u: the kk[u]-th largest score of row u (the smallest causal score when
    # the whole row is taken)
    kmax = int(kk.max())
    part = -np.partition(-s, kmax - 1, axis=1)[:, :kmax]
    t = np.sort(part, axis=1)[:, ::-1][u, kk - 1]
    # the oracle's set: every score above t, then the lowest-indexed ties
    gt = s > t[:, None]
    eq = (s == t[:, None]) & causal
    need = kk - gt.sum(axis=1)
    ref = gt | (eq & (np.cumsum(eq, axis=1) <= need[:, None]))
    diff = ref ^ sel
    with np.errstate(invalid="ignore"):
        near = np.abs(s - t[:, None]) <= NEAR_TIE_REL * np.abs(t)[:, None]
    bad = diff & ~near
    assert not bad.any(), (f"{what}: block rows {np.nonzero(bad.any(axis=1))[0][:8].tolist()} "
                           f"differ beyond the near-tie band")
    nd = int(diff.sum())
    return nd, nd


def compare_output(O_gpu, O_ref, dtype, what=""):
    """Element-wise comparison to the benchmark spec's tolerances."""
    d = np.abs(np.asarray(O_gpu, dtype=np.float64) - O_ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    lim = (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == "bf16" else (F32_MAX_ABS, F32_MEAN_ABS)
    log(f"  {what}: max-abs {mx:.3e} (<= {lim[0]:g}), mean-abs {mean:.3e} (<= {lim[1]:g})")
    if d.ndim == 4 and (mx > lim[0] or mean > lim[1] or not np.all(np.isfinite(O_gpu))):
        for b in range(d.shape[0]):
            for h in range(d.shape[1]):
                dr = d[b, h].max(axis=-1)
                bad = np.nonzero(dr > lim[0])[0]
                log(f"    head ({b},{h}): max-abs {dr.max():.3e}, {bad.size} rows over, first {bad[:12].tolist()}")
    assert np.all(np.isfinite(O_gpu)), f"{what}: non-finite output"
    assert mx <= lim[0], f"{what}: max-abs {mx} > {lim[0]}"
    assert mean <= lim[1], f"{what}: mean-abs {mean} > {lim[1]}"
    return mx, mean


def check_selection(gpu_idx, scores, k, what):
    """GPU top-k vs the oracle's: identical except candidates whose oracle
    score lies within 1e-4 relative of the k-th threshold.  Returns
    (number of differences, number exempt)."""
    g = np.asarray(gpu_idx, dtype=np.int64)
    g = g[g >= 0]
    k = min(int(k), scores.shape[0])
    assert g.shape[0] == k, f"{what}: {g.shape[0]} indices, expected {k}"
    assert np.all(np.diff(g) > 0), f"{what}: not strictly ascending"
    ref = O.topk_ascending(scores, k)
    if k == 0:
        return 0, 0
    t = O.kth_threshold(scores, k)
    diff = np.setxor1d(g, ref)
    near = np.abs(scores[diff] - t) <= NEAR_TIE_REL * abs(t)
    assert np.all(near), f"{what}: {int((~near).sum())} selections differ beyond the near-tie band"
    return int(diff.shape[0]), int(near.sum())


def check_tiles(p, res, buf):
    """Exact checks of the GPU tile lists against the oracle's index sets.
    The lists are the 64-row slash expansion under either slash_tile (exact
    pairs only add a per-pair test); kept edges follow the oracle run's
    slash_tile."""
    slash_tile = 64
    sz = buf["sizes"]
    t = {k: v.cpu().numpy() for k, v in buf["tiles"].items()}
    n, nq = p.n, int(sz.nq)
    assert t["status"][0] == 0, f"device status {t['status'][0]}"
    for (b, h), r in res["heads"].items():
        assert int(t["kept_edges"][b, h]) == r.edges, f"kept edges of head ({b},{h}): {t['kept_edges'][b, h]} vs {r.edges}"
        if r.kind != O.VSLASH:
            continue
        cover = O.slash_offset_set(r.offs, n, slash_tile)            # x + 63
        ns = int(t["span_cnt"][b, h])
        lo, hi = t["span_lo"][b, h, :ns], t["span_hi"][b, h, :ns]
        got = np.zeros_like(cover)
        for a, e in zip(lo, hi):
            assert a <= e and a >= -63 and e < n
            got[a + 63:e + 64] = True
        assert np.array_equal(got, cover), f"span set of head ({b},{h})"
        assert np.all(lo[1:] > hi[:-1] + 1), "spans not disjoint / merged"
        # the whole 32-offset chunks (ascending) and the packed tail offsets
        # hold each span offset once; block u uses the chunks and packed
        # chunks that start at or below 64u, which hold every span offset
        # x <= 64u
        clo, chi = t["chunk_lo"][b, h], t["chunk_hi"][b, h]
        used = int(t["chunk_cnt"][b, h, nq - 1])      # chunks of the last block
        assert np.all(np.diff(clo[:used]) > 0), "chunks not ascending"
        # tails are packed unless under exact slash pairs (slash_tile == 1)
        packed = int(sz.bits_words) == 0
        for a, e in zip(clo[:used], chi[:used]):
            assert (e - a == 31) if packed else (0 <= e - a <= 31), "chunk width"
        tcnt = int(t["tail_cnt"][b, h])
        tx = t["tail_x"][b, h]
        if not packed:
            assert tcnt == 0, "unpacked tails stay chunks of their own"
        assert np.all(np.diff(tx[:tcnt]) > 0), "tail offsets not ascending"
        npk = (tcnt + 31) // 32
        assert np.all(tx[tcnt:32 * npk] == M.MINF_TAIL_PAD), "tail padding"
        chunk_x = np.concatenate([np.arange(a, e + 1) for a, e in zip(clo[:used], chi[:used])] +
                                 [np.zeros(0, np.int64)])
        both = np.concatenate([chunk_x, tx[:tcnt]])
        assert len(np.unique(both)) == len(both), "an offset in two chunks"
        got2 = np.zeros_like(cover)
        got2[both + 63] = True
        X = 64 * (nq - 1)
        assert not np.any(got2 & ~cover), "a chunk leaves the spans"
        assert np.array_equal(got2[:X + 64], cover[:X + 64]), "chunks miss part of the spans"
        nch = np.array([int(np.sum(clo[:used] <= 64 * u)) for u in range(nq)])
        assert np.array_equal(t["chunk_cnt"][b, h].astype(np.int64), nch), "chunk counts"
        firsts = tx[0:32 * npk:32]
        npk_u = np.array([int(np.sum(firsts <= 64 * u)) for u in range(nq)])
        assert np.array_equal(t["pk_cnt"][b, h].astype(np.int64), npk_u), "packed chunk counts"
        # every covered offset x <= 64u lies in a chunk or packed chunk that
        # block u uses
        cl = np.concatenate([[0], np.cumsum(chi[:used] - clo[:used] + 1)])
        for u in range(nq):
            act = np.concatenate([chunk_x[:cl[nch[u]]], tx[:min(tcnt, 32 * npk_u[u])]])
            want = np.nonzero(cover[:64 * u + 64])[0] - 63
            assert np.all(np.isin(want, act)), f"block {u} misses a span offset"
        cols = np.asarray(r.cols, dtype=np.int64)
        for u in range(nq):
            end = min(64 * u + 63, n - 1)
            c = cols[cols <= end]
            exp = c[~cover[64 * u - c + 63]]
            cc = int(t["col_cnt"][b, h, u])
            assert np.array_equal(t["cols"][b, h, u, :cc], exp), f"columns of ({b},{h}) block {u}"


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  [{self.what}: {time.time() - self.t:.1f}s]")
