"""Seeded synthetic inputs for MInference-style sparse prefill.

This module only draws numbers: Q, K, V tensors, the per-head pattern table and
the sampled query rows.  It holds none of the attention, index or tile
arithmetic, so both the CPU oracle and the GPU path can take their inputs from
here without sharing any of the method's code.

Shapes follow the pages' own layout (PaperTrace "2.1.2 MInference", section 1.1):
Q is [B, Hq, n, dh], K and V are [B, Hkv, n, dh], contiguous.  Half-precision
tensors are returned as raw bfloat16 bit patterns (numpy uint16), fp32 tensors
as numpy float32.

Recipe (fixed before any measurement):

* Workload ``k`` (1..5) is seeded with ``1000 + k``.
  ``SeedSequence(seed).spawn(6)`` gives, in order, the streams for Q, K, V, the
  planted structure, the pattern table and the sampled rows.  The Q, K and V
  streams are further spawned into one child per head so heads can be drawn in
  parallel; every stream feeds a ``Generator(PCG64)``.
* Normals are drawn in float64 and rounded once to the target type
  (round-to-nearest-even; for bfloat16 via round-to-odd float32, which makes
  the two-step rounding exact).
* "Planted" distribution (the 32K, 128K and 1M workloads): i.i.d. N(0,1) plus
  16 attention-sink keys shared by all heads and a periodic relative-offset
  comb (period P=1024, H=16 harmonics), each worth +3 sigma of the logit
  q.k/sqrt(dh).  The sinks stand in for the anchor tokens and the comb for the
  "periodic structure, paragraph spacing" slashes the MInference pages describe.
* "Clustered" distribution (the 512K workload): 256 Gaussian centres per KV
  head, tokens assigned to clusters in runs of 32..512 positions, noise
  sigma 0.5; V is N(0,1).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# Pattern kinds.  These codes are part of the library's C interface
# (minf_kind in include/minf.h) and of the oracle's input format.
ASHAPE = 0
VSLASH = 1
BSPARSE = 2
KIND_NAMES = {ASHAPE: "ashape", VSLASH: "vslash", BSPARSE: "bsparse"}

FORCE_FIRST_BLOCK = 1
FORCE_DIAG_BLOCK = 2

BLOCK = 64


@dataclass
class HeadCfg:
    """One query head's entry in the layer's pattern table (PaperTrace 2.1.2,
    section 6.3: kind plus vertical/slash counts, block budget, window and
    initial tokens)."""
    kind: int
    sink: int = 0
    window: int = 0
    last_q: int = 0
    n_vertical: int = 0
    n_slash: int = 0
    topk_blocks: int = 0
    force_flags: int = 0

    def as_tuple(self):
        return (self.kind, self.sink, self.window, self.last_q, self.n_vertical,
                self.n_slash, self.topk_blocks, self.force_flags)


def ashape(sink, window):
    return HeadCfg(ASHAPE, sink=sink, window=window)


def vslash(last_q, n_vertical, n_slash):
    return HeadCfg(VSLASH, last_q=last_q, n_vertical=n_vertical, n_slash=n_slash)


def bsparse(topk, force=0):
    return HeadCfg(BSPARSE, topk_blocks=topk, force_flags=force)


@dataclass
class Problem:
    name: str
    B: int
    Hq: int
    Hkv: int
    n: int
    dh: int
    dtype: str                     # "f32" or "bf16"
    heads: List[HeadCfg]
    Q: np.ndarray                  # float32 or uint16 (bf16 bits)
    K: np.ndarray
    V: np.ndarray
    scale: float = 0.0             # 0 means 1/sqrt(dh)
    rows: Optional[np.ndarray] = None   # sampled query rows, or None = all rows
    edge_rows: Optional[np.ndarray] = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def eff_scale(self):
        return self.scale if self.scale else 1.0 / math.sqrt(self.dh)


# --------------------------------------------------------------------------
# rounding helpers (input preparation only)
# --------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Correctly rounded (nearest-even) float64 -> bfloat16 bit patterns.

    float64 is first rounded to float32 with round-to-odd, then float32 to
    bfloat16 with round-to-nearest-even; since float32 keeps more than
    bfloat16's 8 bits + 2, the composition equals one correct rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    t = x.astype(np.float32)                      # RNE
    back = t.astype(np.float64)
    over = np.abs(back) > np.abs(x)               # rounded away from zero
    t = np.where(over, np.nextafter(t, np.float32(0)), t)
    bits = t.view(np.uint32).copy()
    inexact = t.astype(np.float64) != x
    bits |= inexact.astype(np.uint32)             # sticky (odd) bit
    rnd = ((bits >> 16) & 1) + np.uint32(0x7FFF)
    return ((bits + rnd) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    return x.astype(np.float32)


def _workers(workers):
    if workers:
        return workers
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:
        c = os.cpu_count() or 1
    return max(1, min(16, c))


# --------------------------------------------------------------------------
# distributions
# --------------------------------------------------------------------------

def _planted_structure(rng, Hkv, n, dh, n_sinks=16, period=1024, harmonics=16):
    """Sink positions and per-KV-head orthonormal directions."""
    sinks = np.sort(rng.choice(n, size=min(n_sinks, n), replace=False)).astype(np.int64)
    dirs = []
    ncols = 1 + 2 * harmonics
    assert ncols <= dh
    for _ in range(Hkv):
        g = rng.standard_normal((dh, ncols))
        qm, r = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(r))[None, :]     # unique orientation
        dirs.append(qm)                            # [dh, 1+2H]
    return sinks, dirs


def _comb_features(pos: np.ndarray, period: int, harmonics: int) -> np.ndarray:
    """[len(pos), 2H] matrix of cos(m theta p), sin(m theta p), m = 1..H."""
    theta = 2.0 * math.pi / period
    m = np.arange(1, harmonics + 1, dtype=np.float64)
    ang = (pos.astype(np.float64) % period)[:, None] * m[None, :] * theta
    f = np.empty((pos.shape[0], 2 * harmonics))
    f[:, 0::2] = np.cos(ang)
    f[:, 1::2] = np.sin(ang)
    return f


def _planted_tensor(seed_seq, n, dh, dirs_k, sinks, is_key, dtype,
                    period, harmonics, sink_amp, comb_amp):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    out = np.empty((n, dh), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 16
    # dirs_k columns: [u, e1_1, e2_1, e1_2, e2_2, ...]
    u = dirs_k[:, 0]
    comb_dirs = dirs_k[:, 1:]                      # [dh, 2H], interleaved (e1_m, e2_m)
    for s in range(0, n, step):
        e = min(n, s + step)
        x = rng.standard_normal((e - s, dh))
        pos = np.arange(s, e)
        x += comb_amp * (_comb_features(pos, period, harmonics) @ comb_dirs.T)
        if is_key:
            sel = sinks[(sinks >= s) & (sinks < e)]
            if sel.size:
                x[sel - s] += sink_amp * u[None, :]
        else:
            x += sink_amp * u[None, :]
        out[s:e] = _round(x, dtype)
    return out


def _local_features(pos: np.ndarray, harmonics: int, lmin: float = 32.0, lmax: float = 4096.0) -> np.ndarray:
    """[len(pos), 2H] matrix of cos, sin of 2 pi p / L_m for H wavelengths L_m
    spaced geometrically from lmin to lmax: their dot product between
    positions i and j is sum_m cos(2 pi (i - j) / L_m), largest at i = j."""
    m = np.arange(harmonics, dtype=np.float64)
    lam = lmin * (lmax / lmin) ** (m / max(harmonics - 1, 1))
    ang = pos.astype(np.float64)[:, None] * (2.0 * math.pi / lam)[None, :]
    f = np.empty((pos.shape[0], 2 * harmonics))
    f[:, 0::2] = np.cos(ang)
    f[:, 1::2] = np.sin(ang)
    return f


def _local_tensor(seed_seq, n, dh, dirs_k, n_sinks, is_key, dtype, harmonics, sink_amp, amp):
    """Local structure: iid noise plus positional features that make q_i . k_j
    peak near i = j, and the first n_sinks keys raised along a direction that
    every query shares (the sink of an A-shape head)."""
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    out = np.empty((n, dh), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 16
    u = dirs_k[:, 0]
    feat_dirs = dirs_k[:, 1:]
    for s in range(0, n, step):
        e = min(n, s + step)
        x = rng.standard_normal((e - s, dh))
        x += amp * (_local_features(np.arange(s, e), harmonics) @ feat_dirs.T)
        if is_key:
            if s < n_sinks:
                x[:min(n_sinks, e) - s] += sink_amp * u[None, :]
        else:
            x += sink_amp * u[None, :]
        out[s:e] = _round(x, dtype)
    return out


def _iid_tensor(seed_seq, n, dh, dtype):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    out = np.empty((n, dh), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 16
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = _round(rng.standard_normal((e - s, dh)), dtype)
    return out


def _clustered_tensor(seed_seq, centres, ids, sigma, dtype):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    n = ids.shape[0]
    dh = centres.shape[1]
    out = np.empty((n, dh), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 16
    for s in range(0, n, step):
        e = min(n, s + step)
        x = centres[ids[s:e]] + sigma * rng.standard_normal((e - s, dh))
        out[s:e] = _round(x, dtype)
    return out


def _cluster_runs(rng, n, n_clusters, lo=32, hi=512):
    ids = np.empty(n, dtype=np.int64)
    p = 0
    while p < n:
        L = int(rng.integers(lo, hi + 1))
        c = int(rng.integers(0, n_clusters))
        ids[p:p + L] = c
        p += L
    return ids


CALIB_KINDS = ("local", "planted", "clustered")


def _sample_rows(rng, n, count=4096):
    if count >= n:
        return np.arange(n, dtype=np.int64)
    return np.sort(rng.choice(n, size=count, replace=False)).astype(np.int64)


def _edge_rows(n):
    cand = [0, 1, 63, 64, 65, n // 2, n - 65, n - 64, n - 1]
    return np.array(sorted({c for c in cand if 0 <= c < n}), dtype=np.int64)


def generate(name, B, Hq, Hkv, n, dh, dtype, heads, seed, dist="iid",
             scale=0.0, sample_rows=None, workers=None,
             period=1024, harmonics=16, n_sinks=16,
             n_clusters=256, cluster_sigma=0.5):
    """Draw one problem.

    dist: "iid" (N(0,1)), "planted" (sinks + periodic comb), "clustered", or
          "calibration": KV group kv takes the structure CALIB_KINDS[kv % 3]
          (local, planted or clustered), so that the heads of one layer want
          different patterns.
    sample_rows: None to check every row, else the number of sampled rows.
    """
    assert Hq % Hkv == 0 and len(heads) == Hq
    root = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_struct, s_pat, s_rows = root.spawn(6)
    g = Hq // Hkv
    q_seeds = s_q.spawn(B * Hq)
    k_seeds = s_k.spawn(B * Hkv)
    v_seeds = s_v.spawn(B * Hkv)
    st = np.random.Generator(np.random.PCG64(s_struct))
    meta = {"dist": dist}
    jobs = []
    Q = np.empty((B, Hq, n, dh), dtype=np.uint16 if dtype == "bf16" else np.float32)
    K = np.empty((B, Hkv, n, dh), dtype=Q.dtype)
    V = np.empty((B, Hkv, n, dh), dtype=Q.dtype)

    if dist == "planted":
        sink_amp = math.sqrt(3.0 * math.sqrt(dh))
        comb_amp = math.sqrt(3.0 * math.sqrt(dh) / harmonics)
        per_batch = []
        for b in range(B):
            per_batch.append(_planted_structure(st, Hkv, n, dh, n_sinks, period, harmonics))
        meta.update(period=period, harmonics=harmonics, sink_amp=sink_amp,
                    comb_amp=comb_amp, sinks=[pb[0] for pb in per_batch])
        for b in range(B):
            sinks, dirs = per_batch[b]
            for h in range(Hq):
                jobs.append((Q, (b, h), _planted_tensor,
                             (q_seeds[b * Hq + h], n, dh, dirs[h // g], sinks, False,
                              dtype, period, harmonics, sink_amp, comb_amp)))
            for kv in range(Hkv):
                jobs.append((K, (b, kv), _planted_tensor,
                             (k_seeds[b * Hkv + kv], n, dh, dirs[kv], sinks, True,
                              dtype, period, harmonics, sink_amp, comb_amp)))
                jobs.append((V, (b, kv), _iid_tensor, (v_seeds[b * Hkv + kv], n, dh, dtype)))
    elif dist == "clustered":
        per_batch = []
        for b in range(B):
            centres = [st.standard_normal((n_clusters, dh)) for _ in range(Hkv)]
            ids = _cluster_runs(st, n, n_clusters)
            per_batch.append((centres, ids))
        meta.update(n_clusters=n_clusters, sigma=cluster_sigma)
        for b in range(B):
            centres, ids = per_batch[b]
            for h in range(Hq):
                jobs.append((Q, (b, h), _clustered_tensor,
                             (q_seeds[b * Hq + h], centres[h // g], ids, cluster_sigma, dtype)))
            for kv in range(Hkv):
                jobs.append((K, (b, kv), _clustered_tensor,
                             (k_seeds[b * Hkv + kv], centres[kv], ids, cluster_sigma, dtype)))
                jobs.append((V, (b, kv), _iid_tensor, (v_seeds[b * Hkv + kv], n, dh, dtype)))
    elif dist == "calibration":
        sink_amp = math.sqrt(3.0 * math.sqrt(dh))
        comb_amp = math.sqrt(3.0 * math.sqrt(dh) / harmonics)
        # local: q_i . k_i / sqrt(dh) is about 24 from the positional
        # features, against a spread of about 24 / sqrt(2 harmonics) far
        # from the diagonal, so that little mass lies beyond a few thousand
        # keys even at long lengths
        local_amp = math.sqrt(24.0 * math.sqrt(dh) / harmonics)
        kinds = [CALIB_KINDS[kv % 3] for kv in range(Hkv)]
        meta.update(group_kinds=kinds, period=period, harmonics=harmonics)
        for b in range(B):
            sinks, dirs = _planted_structure(st, Hkv, n, dh, n_sinks, period, harmonics)
            centres = [st.standard_normal((n_clusters, dh)) for _ in range(Hkv)]
            ids = _cluster_runs(st, n, n_clusters)
            for kv in range(Hkv):
                kind = kinds[kv]
                heads_kv = range(kv * g, (kv + 1) * g)
                if kind == "local":
                    for h in heads_kv:
                        jobs.append((Q, (b, h), _local_tensor, (q_seeds[b * Hq + h], n, dh, dirs[kv], 4, False,
                                                                 dtype, harmonics, sink_amp, local_amp)))
                    jobs.append((K, (b, kv), _local_tensor, (k_seeds[b * Hkv + kv], n, dh, dirs[kv], 4, True,
                                                              dtype, harmonics, sink_amp, local_amp)))
                elif kind == "planted":
                    for h in heads_kv:
                        jobs.append((Q, (b, h), _planted_tensor,
                                     (q_seeds[b * Hq + h], n, dh, dirs[kv], sinks, False,
                                      dtype, period, harmonics, sink_amp, comb_amp)))
                    jobs.append((K, (b, kv), _planted_tensor,
                                 (k_seeds[b * Hkv + kv], n, dh, dirs[kv], sinks, True,
                                  dtype, period, harmonics, sink_amp, comb_amp)))
                else:
                    for h in heads_kv:
                        jobs.append((Q, (b, h), _clustered_tensor,
                                     (q_seeds[b * Hq + h], centres[kv], ids, cluster_sigma, dtype)))
                    jobs.append((K, (b, kv), _clustered_tensor,
                                 (k_seeds[b * Hkv + kv], centres[kv], ids, cluster_sigma, dtype)))
                jobs.append((V, (b, kv), _iid_tensor, (v_seeds[b * Hkv + kv], n, dh, dtype)))
    elif dist == "iid":
        for b in range(B):
            for h in range(Hq):
                jobs.append((Q, (b, h), _iid_tensor, (q_seeds[b * Hq + h], n, dh, dtype)))
            for kv in range(Hkv):
                jobs.append((K, (b, kv), _iid_tensor, (k_seeds[b * Hkv + kv], n, dh, dtype)))
                jobs.append((V, (b, kv), _iid_tensor, (v_seeds[b * Hkv + kv], n, dh, dtype)))
    else:
        raise ValueError(dist)

    def run(job):
        dst, idx, fn, args = job
        dst[idx] = fn(*args)

    nw = _workers(workers)
    if nw == 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(run, jobs))

    rr = np.random.Generator(np.random.PCG64(s_rows))
    rows = None if sample_rows is None else _sample_rows(rr, n, sample_rows)
    return Problem(name=name, B=B, Hq=Hq, Hkv=Hkv, n=n, dh=dh, dtype=dtype,
                   heads=list(heads), Q=Q, K=K, V=V, scale=scale, rows=rows,
                   edge_rows=_edge_rows(n), seed=seed, meta=meta)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

VS_STD = dict(last_q=64, n_vertical=1000, n_slash=6096)

WORKLOADS = {
    1: dict(name="n2048_h4_d64_f32_mixed", B=1, Hq=4, Hkv=4, n=2048, dh=64, dtype="f32", dist="iid"),
    2: dict(name="n32k_h32kv8_d128_bf16_vs", B=1, Hq=32, Hkv=8, n=32768, dh=128, dtype="bf16", dist="planted"),
    3: dict(name="n128k_h32kv8_d128_bf16_mixed", B=1, Hq=32, Hkv=8, n=131072, dh=128, dtype="bf16", dist="planted"),
    4: dict(name="n512k_h32kv8_d128_bf16_bs", B=1, Hq=32, Hkv=8, n=524288, dh=128, dtype="bf16", dist="clustered"),
    5: dict(name="n1m_h32kv8_d128_bf16_vs", B=1, Hq=32, Hkv=8, n=1048576, dh=128, dtype="bf16", dist="planted"),
}


def pattern_table(k: int, seed: Optional[int] = None) -> List[HeadCfg]:
    """Per-head pattern table of workload k (the pattern-table stream decides
    the head permutation of the mixed 128K layer)."""
    if k == 1:
        # head 3 is the dense check: block-sparse with every causal block kept
        return [ashape(64, 256), vslash(64, 64, 128), bsparse(16), bsparse(32)]
    if k in (2, 5):
        return [vslash(**VS_STD) for _ in range(32)]
    if k == 3:
        seed = 1000 + k if seed is None else seed
        s_pat = np.random.SeedSequence(seed).spawn(6)[4]
        perm = np.random.Generator(np.random.PCG64(s_pat)).permutation(32)
        heads = [None] * 32
        for r, h in enumerate(perm):
            if r < 16:
                heads[h] = vslash(**VS_STD)
            elif r < 24:
                heads[h] = bsparse(100)
            else:
                heads[h] = ashape(128, 4096)
        return heads
    if k == 4:
        return [bsparse(256, FORCE_FIRST_BLOCK | FORCE_DIAG_BLOCK) for _ in range(32)]
    raise ValueError(k)


def make_workload(k: int, seed: Optional[int] = None, workers=None) -> Problem:
    w = WORKLOADS[k]
    seed = 1000 + k if seed is None else seed
    heads = pattern_table(k, seed)
    sample = None if w["n"] <= 32768 else 4096
    return generate(w["name"], w["B"], w["Hq"], w["Hkv"], w["n"], w["dh"], w["dtype"],
                    heads, seed, dist=w["dist"], sample_rows=sample, workers=workers)


def make_small(n=1000, B=1, Hq=8, Hkv=2, dh=128, dtype="bf16", heads=None,
               seed=7, dist="planted", scale=0.0, workers=None, **kw) -> Problem:
    """A small mixed-pattern problem the oracle finishes in seconds."""
    if heads is None:
        base = [ashape(16, 100), vslash(64, 40, 60), bsparse(4),
                vslash(32, 10, 30), bsparse(3, FORCE_FIRST_BLOCK | FORCE_DIAG_BLOCK),
                ashape(0, 200), vslash(64, 200, 8), bsparse(100)]
        heads = [base[h % len(base)] for h in range(Hq)]
    if dist == "planted":
        kw.setdefault("period", 128)
        kw.setdefault("harmonics", 8)
        kw.setdefault("n_sinks", 4)
    return generate(f"small_n{n}_b{B}_h{Hq}kv{Hkv}_d{dh}_{dtype}", B, Hq, Hkv, n, dh, dtype,
                    heads, seed, dist=dist, scale=scale, workers=workers, **kw)


def make_calibration(n=16384, B=1, Hq=32, Hkv=8, dh=128, dtype="bf16", seed=2024, period=1024, harmonics=16,
                     n_sinks=16, n_clusters=16, workers=None) -> Problem:
    """A calibration layer for the pattern search: KV groups cycle through
    local, planted and clustered structure (CALIB_KINDS); few clusters, so
    that a clustered head's keys recur in blocks across the whole sequence.
    The pattern table it carries is a placeholder (every head dense); the
    search replaces it."""
    heads = [ashape(0, n)] * Hq
    return generate(f"calib_n{n}_h{Hq}kv{Hkv}_d{dh}_{dtype}", B, Hq, Hkv, n, dh, dtype, heads, seed,
                    dist="calibration", period=period, harmonics=harmonics, n_sinks=n_sinks,
                    n_clusters=n_clusters, workers=workers)
