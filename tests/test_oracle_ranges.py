"""Pins of the oracle's row-by-row attention over key ranges (oracle/attend.c
and the range lists of minf_oracle.py), which the full-size parity checks use
at long sequences.

* The range lists of every pattern give, row by row, exactly the candidate
  sets of the masks (Eq. 3, Eq. 6, the slash expansion and Eq. 5), which the
  loop brute force pins;
* the C restricted softmax equals the vectorised oracle's to 1e-12 on every
  row, the loop-only brute force (oracle/brute.py) on tiny inputs, and
  torch's scaled_dot_product_attention in float64 for dense causal ranges
  (MInference page, section 1.1, Eq. 1-2);
* an empty candidate set gives o = 0 and LSE = -inf.
"""
import math

import numpy as np
import torch

from oracle import brute
from oracle import minf_oracle as O
from synth import gen


def _keys(lo, hi):
    out = [np.arange(a, b + 1) for a, b in zip(lo, hi) if a <= b]
    k = np.concatenate(out) if out else np.zeros(0, dtype=np.int64)
    assert np.unique(k).shape[0] == k.shape[0], "ranges overlap"
    return np.sort(k)


def test_ranges_equal_masks():
    rng = np.random.default_rng(5)
    n = 333
    rows = np.arange(n)
    for g, w in [(0, 1), (4, 16), (64, 0), (0, n), (100, 50), (3, 1)]:
        m = O.ashape_mask(rows, n, g, w)
        for i in rows:
            assert np.array_equal(_keys(*O.ashape_row_ranges(int(i), g, w)), np.nonzero(m[i])[0]), (g, w, i)
    nq = O.n_blocks(n)
    J = [np.sort(rng.choice(u + 1, min(3, u + 1), replace=False)) for u in range(nq)]
    m = O.bs_mask(rows, n, J)
    for i in rows:
        assert np.array_equal(_keys(*O.bs_row_ranges(int(i), J)), np.nonzero(m[i])[0]), i
    for t in (64, 1, 8):
        offs = np.sort(rng.choice(n, 9, replace=False))
        cols = np.sort(rng.choice(n, 11, replace=False))
        cover = O.slash_offset_set(offs, n, t)
        m = O.vs_mask(rows, n, n, cols, offs, t, cover)
        runs = O.span_runs(cover, t)
        for i in rows:
            assert np.array_equal(_keys(*O.vs_row_ranges(int(i), cols, cover, t, runs)), np.nonzero(m[i])[0]), (t, i)


def test_c_attention_equals_vectorised_oracle():
    p = gen.make_small(n=300, Hq=4, Hkv=2, dh=64, seed=17,
                       heads=[gen.ashape(16, 40), gen.vslash(32, 8, 12), gen.bsparse(2, gen.FORCE_FIRST_BLOCK),
                              gen.vslash(8, 3, 0)])
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, workers=1)
    sc = p.eff_scale
    rows = np.arange(p.n)
    for h in range(p.Hq):
        r = res["heads"][(0, h)]
        f32 = lambda x: O.widen(x, p.dtype).astype(np.float32)
        q, k, v = f32(p.Q[0, h]), f32(p.K[0, h // 2]), f32(p.V[0, h // 2])
        cfg = p.heads[h]
        if r.kind == O.ASHAPE:
            fn = lambda i: O.ashape_row_ranges(i, cfg.sink, cfg.window)
        elif r.kind == O.BSPARSE:
            fn = lambda i: O.bs_row_ranges(i, r.J)
        else:
            cover = O.slash_offset_set(r.offs, p.n, 64)
            fn = lambda i: O.vs_row_ranges(i, r.cols, cover, 64)
        o, lse = O.attend_rows_ranges(q[rows], k, v, rows, fn, sc)
        assert np.abs(o - res["O"][0, h]).max() < 1e-12
        fin = np.isfinite(res["LSE"][0, h])
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse[fin] - res["LSE"][0, h][fin]).max(initial=0) < 1e-12
        assert np.all(o[~fin] == 0)


def test_c_attention_equals_brute_force():
    n, dh = 70, 6
    heads = [gen.ashape(3, 9), gen.vslash(5, 4, 6), gen.bsparse(1, gen.FORCE_DIAG_BLOCK)]
    p = gen.generate("tiny", 1, 3, 1, n, dh, "f32", heads, seed=41, dist="iid")
    sc = 1 / math.sqrt(dh)
    k, v = np.asarray(p.K[0, 0], dtype=np.float32), np.asarray(p.V[0, 0], dtype=np.float32)
    for h, cfg in enumerate(heads):
        q = np.asarray(p.Q[0, h], dtype=np.float32)
        br = brute.head(q.astype(np.float64).tolist(), k.astype(np.float64).tolist(), v.astype(np.float64).tolist(),
                        cfg.as_tuple(), sc)
        if cfg.kind == O.ASHAPE:
            fn = lambda i: O.ashape_row_ranges(i, cfg.sink, cfg.window)
        elif cfg.kind == O.BSPARSE:
            fn = lambda i: O.bs_row_ranges(i, [np.asarray(x) for x in br["J"]])
        else:
            cover = O.slash_offset_set(np.asarray(br["offs"]), n, 64)
            fn = lambda i: O.vs_row_ranges(i, np.asarray(br["cols"]), cover, 64)
        o, lse = O.attend_rows_ranges(q, k, v, np.arange(n), fn, sc)
        assert np.abs(o - np.array(br["o"])).max() < 1e-12, h
        blse = np.array(br["lse"])
        fin = np.isfinite(blse)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse[fin] - blse[fin]).max(initial=0) < 1e-12


def test_c_dense_ranges_equal_sdpa():
    rng = np.random.default_rng(8)
    n, dh = 200, 32
    q, k, v = (rng.standard_normal((n, dh)).astype(np.float32) for _ in range(3))
    sc = 0.3
    o, lse = O.attend_rows_ranges(q, k, v, np.arange(n),
                                  lambda i: (np.array([0]), np.array([i])), sc)
    t = lambda x: torch.from_numpy(x.astype(np.float64))[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=sc)[0, 0].numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_c_empty_rows():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((10, 8)).astype(np.float32) for _ in range(3))
    empty = lambda i: (np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64))
    o, lse = O.attend_rows_ranges(q[[2, 5]], k, v, np.array([2, 5]), empty, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
