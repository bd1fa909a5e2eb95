"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test names what it pins.  None of them re-types the oracle's formula:
they compare it with printed values, closed forms, invariants, library
routines, or an independent formulation.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import minf_oracle as O

RNG = np.random.default_rng(12345)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example

def _worked(golden_dir):
    g = _load(golden_dir, "vs_worked_example.json")
    n, dh = g["n"], g["dh"]
    q = np.zeros((n, dh)); k = np.zeros((n, dh)); v = np.zeros((n, dh))
    q[g["row"]] = g["q6"]
    for j, x in g["k"].items():
        k[int(j)] = x
    for j, x in g["v"].items():
        v[int(j)] = x
    return g, q, k, v


def test_worked_example_set_and_output(golden_dir):
    """PaperTrace 2.1.2 section 4, Eq. 9-11: N(6) = {1,4,6}, o_6 = (1.266, 0.732)."""
    g, q, k, v = _worked(golden_dir)
    n, t = g["n"], g["slash_tile"]
    mask = O.vs_mask(np.array([g["row"]]), n, n, g["cols"], g["offs"], t)[0]
    assert sorted(np.nonzero(mask)[0].tolist()) == g["expected_set"]
    sc = [float(q[g["row"]] @ k[j]) for j in g["expected_set"]]
    assert sc == g["expected_scores"]
    o, lse = O.attend_rows(q, k, v, np.array([g["row"]]),
                           lambda rr, nk: O.vs_mask(rr, nk, n, g["cols"], g["offs"], t), g["scale"])
    assert np.allclose(o[0], g["printed_o6"], atol=g["printed_tolerance"], rtol=0)
    e = math.e
    exact = [3 * e / (2 * e + 1), (2 + e) / (2 * e + 1)]
    assert np.allclose(o[0], exact, atol=1e-12, rtol=0)
    assert abs(lse[0] - math.log(2 * e ** 2 + e)) < 1e-12
    w = np.exp(np.array(sc) - lse[0])
    assert np.allclose(w, g["printed_weights"], atol=5e-4)


def test_worked_example_clipping_and_dedup():
    """Same section: offset 2 gives a negative key for row 1 and is dropped;
    a key reached by both a vertical and a slash is counted once."""
    n = 8
    m1 = O.vs_mask(np.array([1]), n, n, [1], [0, 2], 1)[0]
    assert np.nonzero(m1)[0].tolist() == [1]
    m6 = O.vs_mask(np.array([6]), n, n, [6], [0], 1)[0]
    assert np.nonzero(m6)[0].tolist() == [6]
    counts = O.vs_row_counts(n, [6], [0], 1)
    # rows 0..6 keep only their diagonal key (row 6: key 6 once), row 7 keeps 6 and 7
    assert counts.tolist() == [1] * 7 + [2]
    assert O.vs_edges(n, [6], [0], 1) == 9


# ---------------------------------------------------------------- proxy miss example

def test_proxy_miss_example_selection(golden_dir):
    """PaperTrace 2.1.2 section 4.1, Eq. 12: the column statistic picks column 1."""
    g = _load(golden_dir, "proxy_miss_example.json")
    P = np.array(g["P"])
    colmax = P.max(axis=0)
    assert np.allclose(colmax, g["printed_column_max"])
    assert O.topk_ascending(colmax, 1).tolist() == [g["printed_choice_index"]]
    assert np.allclose(P.sum(axis=0), g["column_sum"])
    assert O.topk_ascending(P.sum(axis=0), 1).tolist() == [g["printed_choice_index"]]


# ---------------------------------------------------------------- edge counts

def test_printed_edge_counts(golden_dir):
    """Kept-edge counts printed on the pages (cost model sections 1.2, 2.1,
    2.2, 4.2; MInference Figure 1 and section 4.1)."""
    g = _load(golden_dir, "edge_counts.json")
    for c in g["cases"]:
        n = c["n"]
        if c["kind"] == "dense":
            got = int(O.ashape_row_counts(n, n, 0).sum())           # all initial keys
            got2 = O.bs_edges(n, [np.arange(u + 1) for u in range(O.n_blocks(n))])
            assert got == got2
        elif c["kind"] == "window":
            got = int(O.ashape_row_counts(n, 0, c["window"]).sum())
        elif c["kind"] == "ashape":
            got = int(O.ashape_row_counts(n, c["sink"], c["window"]).sum())
        else:
            got = O.vs_edges(n, c["cols"], c["offs"], 64)
            assert got == O.vs_edges(n, c["cols"], c["offs"], 1)
        assert got == c["edges"], c["what"]


def test_ashape_counts_closed_form():
    """|N_A(i)| = min(i+1, g+w) (the two sets of Eq. 3 overlap only at the
    start), so E_A = n*m - m(m-1)/2 with m = g+w once n >= m."""
    for n, g, w in [(1000, 64, 256), (2048, 64, 256), (300, 0, 17), (50, 60, 10), (131072, 128, 4096)]:
        cnt = O.ashape_row_counts(n, g, w)
        assert np.array_equal(cnt, np.minimum(np.arange(n) + 1, g + w))
        m = g + w
        if n >= m:
            assert int(cnt.sum()) == n * m - m * (m - 1) // 2
    # the 2048-token mixed layer's A-shape head keeps 604,320 edges
    assert int(O.ashape_row_counts(2048, 64, 256).sum()) == 604320


def test_vs_edges_match_row_counts_and_mask():
    """Three independent countings of the VS set agree: per-row masks,
    per-row prefix counts and the block-wise total."""
    for n, t in [(200, 64), (200, 1), (130, 64), (97, 8)]:
        cols = np.sort(RNG.choice(n, 12, replace=False))
        offs = np.sort(RNG.choice(n, 9, replace=False))
        rows = np.arange(n)
        m = O.vs_mask(rows, n, n, cols, offs, t)
        rc = O.vs_row_counts(n, cols, offs, t)
        assert np.array_equal(m.sum(axis=1), rc)
        assert O.vs_edges(n, cols, offs, t) == int(rc.sum())


# ---------------------------------------------------------------- dense attention

def test_dense_matches_torch_sdpa():
    """Dense causal attention reduces to a library routine (torch SDPA, fp64)."""
    import torch
    n, dh = 77, 16
    q, k, v = (RNG.standard_normal((n, dh)) for _ in range(3))
    o, lse = O.dense_attention(q, k, v, 1 / math.sqrt(dh))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        is_causal=True)[0, 0].numpy()
    assert np.abs(o - ref).max() < 1e-12
    s = (q @ k.T) / math.sqrt(dh)
    ref_lse = np.array([np.log(np.exp(s[i, :i + 1]).sum()) for i in range(n)])
    assert np.abs(lse - ref_lse).max() < 1e-12


@pytest.mark.parametrize("n", [50, 129, 200])
def test_full_budgets_reproduce_dense(n):
    """Budgets that cover the whole causal triangle give dense attention:
    A-shape with g+w >= n, VS with all columns or all offsets, BS with every
    causal block."""
    dh = 8
    q, k, v = (RNG.standard_normal((n, dh)) for _ in range(3))
    sc = 0.3
    od, ld = O.dense_attention(q, k, v, sc)
    rows = np.arange(n)
    masks = [
        lambda rr, nk: O.ashape_mask(rr, nk, n // 2, n - n // 2),
        lambda rr, nk: O.ashape_mask(rr, nk, 0, n),
        lambda rr, nk: O.vs_mask(rr, nk, n, np.arange(n), [], 64),
        lambda rr, nk: O.vs_mask(rr, nk, n, [], np.arange(n), 64),
        lambda rr, nk: O.vs_mask(rr, nk, n, [], np.arange(n), 1),
        lambda rr, nk: O.bs_mask(rr, nk, [np.arange(u + 1) for u in range(O.n_blocks(n))]),
    ]
    for mf in masks:
        o, l = O.attend_rows(q, k, v, rows, mf, sc)
        assert np.abs(o - od).max() < 1e-12
        assert np.abs(l - ld).max() < 1e-12
    # and the index step with full budgets selects everything
    J = O.bs_index(q, k, O.n_blocks(n), 0, sc)
    assert all(list(J[u]) == list(range(u + 1)) for u in range(len(J)))
    cols, offs, _, _ = O.vs_index(q, k, 64, n, n, sc)
    assert list(cols) == list(range(n)) and list(offs) == list(range(n))


def test_empty_row_gives_zero():
    n, dh = 20, 4
    q, k, v = (RNG.standard_normal((n, dh)) for _ in range(3))
    # verticals only at 10: rows < 10 have no candidate
    o, l = O.attend_rows(q, k, v, np.arange(n), lambda rr, nk: O.vs_mask(rr, nk, n, [10], [], 1), 1.0)
    assert np.all(o[:10] == 0) and np.all(np.isneginf(l[:10]))
    assert np.allclose(o[10:], v[10])


# ---------------------------------------------------------------- online softmax

def test_online_merge_equals_one_shot():
    """PaperTrace 2.1.2 section 3.2, Eq. 7-8 (and the cost model's section
    3.2): merging tiles with a running max, sum and accumulator gives the
    one-shot softmax the oracle computes, even when a later tile's maximum
    is 80 above the earlier ones."""
    n, dh = 200, 8
    q, k, v = (RNG.standard_normal((n, dh)) for _ in range(3))
    k[150:170] *= 40.0                           # extreme logits in a late tile
    i = n - 1
    keys = np.sort(RNG.choice(i + 1, 120, replace=False))
    keys = np.union1d(keys, np.arange(150, 170))
    o, lse = O.attend_rows(q, k, v, np.array([i]),
                           lambda rr, nk: np.isin(np.arange(nk), keys)[None, :], 1.0)
    x_all = k[keys] @ q[i]
    assert x_all.max() - x_all[keys < 150].max() > 80
    m, l, p = -np.inf, 0.0, np.zeros(dh)
    for part in np.array_split(keys, 7):
        x = k[part] @ q[i]
        m2 = max(m, x.max())
        l = math.exp(m - m2) * l + np.exp(x - m2).sum()
        p = math.exp(m - m2) * p + np.exp(x - m2) @ v[part]
        m = m2
    assert np.abs(o[0] - p / l).max() < 1e-12
    assert abs(lse[0] - (m + math.log(l))) < 1e-12


# ---------------------------------------------------------------- proxies

def test_block_pooling_commutes_with_dot():
    """PaperTrace 2.1.2 section 2 (Block-Sparse) and blog 2.3.2: the mean of
    the raw dot products of a block pair equals the dot product of the
    block means."""
    n, dh = 150, 12
    q, k = RNG.standard_normal((n, dh)), RNG.standard_normal((n, dh))
    r = O.bs_block_scores(q, k, 1.0)
    for u in range(O.n_blocks(n)):
        for vb in range(u + 1):
            blk = q[64 * u:64 * u + 64] @ k[64 * vb:64 * vb + 64].T
            assert abs(blk.mean() - r[u, vb]) < 1e-12
    assert np.all(np.isneginf(r[np.triu_indices(r.shape[0], 1)]))


def test_vs_proxy_mass_and_single_row():
    """Each sampled row's proxy weights form a softmax, so the column scores
    and the diagonal scores each sum to the number of sampled rows; with one
    sampled row they are that row's causal softmax (scipy) read forwards and
    backwards."""
    from scipy.special import softmax
    n, dh = 300, 16
    q, k = RNG.standard_normal((n, dh)), RNG.standard_normal((n, dh))
    for L in (1, 7, 64, 400):
        c, r = O.vs_proxy_scores(q, k, L, 0.25)
        assert abs(c.sum() - min(L, n)) < 1e-9 and abs(r.sum() - min(L, n)) < 1e-9
        assert np.all(c >= 0) and np.all(r >= 0)
    c, r = O.vs_proxy_scores(q, k, 1, 0.25)
    ref = softmax(0.25 * (k @ q[n - 1]))
    assert np.abs(c - ref).max() < 1e-14
    assert np.abs(r - ref[::-1]).max() < 1e-14
    # with two sampled rows, r_0 adds the two diagonal weights
    c, r = O.vs_proxy_scores(q, k, 2, 0.25)
    a1 = softmax(0.25 * (k[:n - 1] @ q[n - 2]))
    a2 = softmax(0.25 * (k @ q[n - 1]))
    assert abs(r[0] - (a1[-1] + a2[-1])) < 1e-14
    assert abs(c[n - 1] - a2[-1]) < 1e-14


def test_topk_ties_against_full_sort():
    """Top-k with exact ties: the lowest index wins; compared with a stable
    full sort."""
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 2.0, -1.0, 2.0])
    assert O.topk_ascending(s, 2).tolist() == [0, 2]
    assert O.topk_ascending(s, 4).tolist() == [0, 2, 3, 4]
    assert O.topk_ascending(s, 100).tolist() == list(range(8))
    for _ in range(50):
        x = RNG.integers(0, 5, size=40).astype(float)
        kk = int(RNG.integers(0, 45))
        ref = sorted(sorted(range(40), key=lambda j: (-x[j], j))[:kk])
        assert O.topk_ascending(x, kk).tolist() == ref
        if kk:
            assert O.kth_threshold(x, kk) == x[ref].min()


def test_slash_tile_one_is_eq5_and_64_is_spans():
    """The prefix-count slash test equals a direct enumeration: with t=1 the
    pairs (i, i-d) of Eq. 5, with t=64 the 64-row tiles around them."""
    n = 150
    cols = [3, 70, 149]
    offs = [0, 5, 66, 130]
    m1 = O.vs_mask(np.arange(n), n, n, cols, offs, 1)
    m64 = O.vs_mask(np.arange(n), n, n, cols, offs, 64)
    for i in range(n):
        eq5 = {c for c in cols if c <= i} | {i - d for d in offs if i - d >= 0}
        assert set(np.nonzero(m1[i])[0].tolist()) == eq5
        u = i // 64
        span = {c for c in cols if c <= i}
        for d in offs:
            span |= {j for j in range(64 * u - d, 64 * u + 64 - d) if 0 <= j <= i}
        assert set(np.nonzero(m64[i])[0].tolist()) == span


def test_row_key_lists_equal_masks_and_row_softmax_equals_attend_rows():
    """The per-row candidate lists (used at long sequence lengths) against the
    dense masks of Eq. 3, 5 and 6, and the per-row softmax against
    attend_rows, on a small problem with ragged n, sinks, windows, slashes
    that run past the start, and forced blocks."""
    rng = np.random.default_rng(11)
    n, dh = 203, 16
    q, k, v = (rng.standard_normal((n, dh)) for _ in range(3))
    sc = 0.3
    rows = np.arange(n)
    # A-shape
    for g, w in [(0, 1), (5, 17), (64, 300), (3, 0)]:
        m = O.ashape_mask(rows, n, g, w)
        for i in (0, 1, 4, 5, 63, 64, 130, 202):
            assert np.array_equal(O.ashape_row_keys(i, g, w), np.nonzero(m[i])[0])
    # Vertical-Slash, both slash readings
    cols = np.sort(rng.choice(n, 17, replace=False))
    offs = np.sort(rng.choice(n, 9, replace=False))
    for t in (64, 1):
        cover = O.slash_offset_set(offs, n, t)
        m = O.vs_mask(rows, n, n, cols, offs, t, cover)
        for i in range(n):
            assert np.array_equal(O.vs_row_keys(i, cols, cover, t), np.nonzero(m[i])[0]), (t, i)
        # row softmax over the list equals the dense restricted softmax
        ref_o, ref_l = O.attend_rows(q, k, v, rows, lambda r, nk: O.vs_mask(r, nk, n, cols, offs, t, cover), sc)
        for i in (0, 7, 64, 150, 202):
            o, l = O.attend_row_keys(q[i], k, v, O.vs_row_keys(i, cols, cover, t), sc)
            assert np.allclose(o, ref_o[i], atol=1e-12) and np.isclose(l, ref_l[i])
    # Block-Sparse with forced blocks and a block list that skips the diagonal
    J = O.bs_index(q, k, 2, O.FORCE_FIRST_BLOCK, sc)
    J[3] = np.array([0, 1])
    m = O.bs_mask(rows, n, J)
    for i in range(n):
        assert np.array_equal(O.bs_row_keys(i, J), np.nonzero(m[i])[0]), i
    # an empty list gives o = 0, LSE = -inf
    o, l = O.attend_row_keys(q[5], k, v, np.zeros(0, dtype=np.int64), sc)
    assert np.all(o == 0) and l == -np.inf
