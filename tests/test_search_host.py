"""Host-side checks of the offline pattern search (PaperTrace 2.1.2
"MInference", sections 3.1 and 6.3; blog-zz7 "LLM模型之MInference", section
2.3.1, Eq. 2): the oracle's error measure and selection rule against closed
forms and hand-worked tables, the search module's selection rule against the
oracle's, and the calibration inputs against the structure they are meant to
carry.  No GPU is needed."""
import math

import numpy as np
import pytest

from oracle import minf_oracle as O
from synth import gen


# ---------------------------------------------------------------- error measure

def test_output_error_hand_example():
    # (1-1)^2 + (2-1)^2 + (3-1)^2 + (4-1)^2 = 14 and |ones|^2 = 4
    d2, r2 = O.output_error(np.array([[[[1.0, 2.0], [3.0, 4.0]]]]), np.ones((1, 1, 2, 2)))
    assert d2.tolist() == [14.0] and r2.tolist() == [4.0]
    assert O.relative_output_error(np.array([[[[1.0, 2.0], [3.0, 4.0]]]]), np.ones((1, 1, 2, 2)))[0] == \
        pytest.approx(math.sqrt(14 / 4))


def test_output_error_closed_forms():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 3, 17, 8))
    # identical outputs: no error; a scaled reference: error |c - 1|, per head
    assert np.all(O.relative_output_error(ref, ref) == 0)
    for c in (0.0, 0.5, 1.25, -1.0):
        assert np.allclose(O.relative_output_error(c * ref, ref), abs(c - 1.0), rtol=1e-12)
    # heads are independent: perturbing head 1 leaves heads 0 and 2 at 0
    a = ref.copy()
    a[:, 1] += 1.0
    e = O.relative_output_error(a, ref)
    assert e[0] == 0 and e[2] == 0 and e[1] > 0
    # the sums run over the batch: two batches of the same error add up
    d2, r2 = O.output_error(a, ref)
    d2b, r2b = O.output_error(a[:1], ref[:1])
    assert np.allclose(d2[1], d2b[1] + O.output_error(a[1:], ref[1:])[0][1])
    # a zero reference: relative error 0 for a zero output, infinite otherwise
    z = np.zeros((1, 2, 3, 4))
    o = z.copy()
    o[0, 1, 0, 0] = 1.0
    assert O.relative_output_error(o, z).tolist() == [0.0, math.inf]


def test_full_budgets_reproduce_dense():
    """With every causal key kept (Vertical-Slash with all columns and
    offsets, Block-Sparse with every causal block, A-shape with a window of
    n), the candidate's output is dense attention: error 0."""
    p = gen.make_calibration(n=300, Hq=3, Hkv=3, dh=32, dtype="f32", period=64, harmonics=4, n_sinks=2,
                             n_clusters=4)
    n, nq = p.n, (p.n + 63) // 64
    dense = O.run_layer(p.Q, p.K, p.V, p.dtype, [gen.ashape(0, n)] * 3)["O"]
    for cfg in (gen.vslash(64, n, n), gen.bsparse(nq), gen.ashape(0, n), gen.ashape(n, 0)):
        out = O.run_layer(p.Q, p.K, p.V, p.dtype, [cfg] * 3)["O"]
        assert np.allclose(O.relative_output_error(out, dense), 0.0, atol=1e-12), cfg
    # a small budget does lose mass on these inputs
    out = O.run_layer(p.Q, p.K, p.V, p.dtype, [gen.ashape(4, 16)] * 3)["O"]
    assert np.all(O.relative_output_error(out, dense) > 1e-3)


# ---------------------------------------------------------------- selection rule

def test_choose_patterns_hand_table():
    times = [1.0, 2.0, 2.0, 5.0]              # candidate 3 plays the dense one
    err = [[0.50, 0.01, 0.00, 0.0],           # 0 fails, 1 is the fastest that passes
           [0.20, 0.20, 0.03, 0.0],           # only 2 and 3 pass: 2 is faster
           [0.01, 0.02, 0.00, 0.0],           # 0 passes and is fastest
           [0.20, 0.04, 0.04, 0.0],           # 1 and 2 tie at 2.0 ms: the earlier one
           [0.20, 0.20, 0.20, 0.0],           # only the dense candidate
           [0.20, 0.20, 0.20, 0.2]]           # nothing passes
    assert O.choose_patterns(err, times, 0.05) == [1, 2, 0, 1, 3, -1]
    # a bound of exactly the error qualifies
    assert O.choose_patterns([[0.05, 0.0]], [1.0, 2.0], 0.05) == [0]


def test_search_rule_matches_oracle_rule():
    """The search module's selection (product host code) and the oracle's,
    written independently, agree on random tables with ties."""
    from long_context_prefill_amd import search as S
    rng = np.random.default_rng(11)
    for _ in range(200):
        H, C = int(rng.integers(1, 9)), int(rng.integers(1, 12))
        err = rng.choice([0.0, 0.01, 0.03, 0.05, 0.08, 0.2], size=(H, C))
        times = rng.choice([0.5, 1.0, 1.5, 2.0], size=C)
        eps = float(rng.choice([0.0, 0.03, 0.05, 0.1]))
        assert S.choose(err.tolist(), times.tolist(), eps) == O.choose_patterns(err, times, eps)


def test_default_grid():
    from long_context_prefill_amd import search as S
    from long_context_prefill_amd import MINF_ASHAPE
    for n in (1000, 16384, 131072):
        g = S.default_grid(n)
        assert g[-1] == S.dense(n) and g.count(S.dense(n)) == 1
        assert {c[0] for c in g[:-1]} <= {0, 1, 2}
        nq = (n + 63) // 64
        for c in g:
            if c[0] == MINF_ASHAPE:
                assert c[2] <= n
            elif c[0] == 1:
                assert c[4] <= n and c[5] <= n
            else:
                assert 1 <= c[6] <= nq
        assert len(set(g)) == len(g)


# ---------------------------------------------------------------- calibration inputs

def test_calibration_structure():
    """The three structure kinds of the calibration layer: local heads keep
    most of their mass near the diagonal, clustered heads in a few key
    blocks, planted heads spread it (columns and diagonals)."""
    p = gen.make_calibration(n=4096, Hq=6, Hkv=3, dh=64, dtype="f32", period=128, harmonics=8, n_sinks=4)
    assert p.meta["group_kinds"] == ["local", "planted", "clustered"]
    n = p.n
    rows = np.arange(n - 256, n)
    stats = []
    for h in range(6):
        q = O.widen(p.Q[0, h], p.dtype)
        k = O.widen(p.K[0, h // 2], p.dtype)
        s = (q[rows] @ k.T) / math.sqrt(p.dh)
        s[np.arange(n)[None, :] > rows[:, None]] = -np.inf
        a = np.exp(s - s.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)
        near = np.mean([a[r, max(0, i - 1023):i + 1].sum() for r, i in enumerate(rows)])
        blocks = np.add.reduceat(a, np.arange(0, n, 64), axis=1)
        top8 = np.sort(blocks, axis=1)[:, ::-1][:, :8].sum(axis=1).mean()
        stats.append((near, top8))
    for h in (0, 1):                          # local
        assert stats[h][0] > 0.5
    for h in (4, 5):                          # clustered
        assert stats[h][1] > 0.9
    for h in (2, 3):                          # planted: neither local nor blocky
        assert stats[h][0] < 0.4 and stats[h][1] < 0.6


# ---------------------------------------------------------------- attention mass

def _tiny():
    p = gen.make_calibration(n=200, Hq=3, Hkv=3, dh=32, dtype="f32", period=64, harmonics=4, n_sinks=2,
                             n_clusters=4)
    return p, 1.0 / math.sqrt(p.dh)


def test_missed_mass_is_half_the_l1_distance_of_eq2():
    """Eq. 2 compares the masked softmax A(M) (renormalised over the kept
    keys) with A_dense; per row their L1 distance is 2 (1 - m)."""
    p, sc = _tiny()
    n = p.n
    rows = np.arange(n)
    for h, cfg in enumerate((gen.ashape(4, 32), gen.vslash(64, 8, 16), gen.bsparse(1))):
        q, k = O.widen(p.Q[0, h], p.dtype), O.widen(p.K[0, h], p.dtype)
        res = O.head_index(q, k, cfg, n, sc)
        m = O.captured_mass(q, k, rows, res.mask_fn, sc)
        causal = np.arange(n)[None, :] <= rows[:, None]
        s = np.where(causal, sc * (q @ k.T), -np.inf)
        dense = np.exp(s - s.max(axis=1, keepdims=True))
        dense /= dense.sum(axis=1, keepdims=True)
        keep = res.mask_fn(rows, n) & causal
        sk = np.where(keep, s, -np.inf)
        mx = sk.max(axis=1, keepdims=True)
        ok = np.isfinite(mx[:, 0])
        a = np.zeros_like(dense)
        a[ok] = np.exp(sk[ok] - mx[ok])
        a[ok] /= a[ok].sum(axis=1, keepdims=True)
        l1 = np.abs(a - dense).sum(axis=1)
        assert np.allclose(l1[ok], 2.0 * (1.0 - m[ok]), atol=1e-12), cfg
        assert 0 < m.min() and m.max() <= 1 + 1e-12


def test_missed_mass_bounds_and_lse_route():
    p, sc = _tiny()
    n = p.n
    nq = (n + 63) // 64
    full = [gen.vslash(64, n, n), gen.bsparse(nq), gen.ashape(0, n)]
    assert np.allclose(O.layer_missed_mass(p.Q, p.K, p.dtype, full), 0.0, atol=1e-12)
    # no kept key at all: nothing captured
    assert np.allclose(O.layer_missed_mass(p.Q, p.K, p.dtype, [gen.ashape(0, 0)] * 3), 1.0)
    # the route the GPU takes: m_i = exp(lse_kept,i - lse_dense,i)
    heads = [gen.ashape(4, 32), gen.vslash(64, 8, 16), gen.bsparse(1)]
    kept = O.run_layer(p.Q, p.K, p.V, p.dtype, heads)
    dense = O.run_layer(p.Q, p.K, p.V, p.dtype, [gen.ashape(0, n)] * 3)
    via_lse = 1.0 - np.exp(kept["LSE"][0] - dense["LSE"][0]).mean(axis=1)
    assert np.allclose(via_lse, O.layer_missed_mass(p.Q, p.K, p.dtype, heads), atol=1e-12)
