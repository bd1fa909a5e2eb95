"""The vectorised oracle against the loop-only brute force on tiny inputs:
every pattern, B=2, GQA group sizes 1, 2 and 4, lengths that are not
multiples of 64, exact ties, and empty rows.

The brute force gets its inputs without the oracle's helpers: the GQA map is
the one the MInference page states (section 5.1: a KV head serves a run of
Hq/Hkv consecutive query heads, h_kv = floor(h / (Hq/Hkv))), written out
here, and bf16 bit patterns are widened by torch.  A wrong map or widening in
the oracle therefore changes its outputs against these."""
import math

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import minf_oracle as O
from synth import gen


def _heads(Hq):
    base = [gen.ashape(3, 9), gen.vslash(5, 4, 6), gen.bsparse(1),
            gen.vslash(64, 2, 3), gen.bsparse(2, gen.FORCE_FIRST_BLOCK | gen.FORCE_DIAG_BLOCK),
            gen.ashape(0, 1), gen.vslash(2, 0, 1), gen.bsparse(1, gen.FORCE_DIAG_BLOCK)]
    return [base[h % len(base)] for h in range(Hq)]


def _gqa(h, Hq, Hkv):
    """KV head of query head h: query heads come in runs of Hq/Hkv per KV head."""
    group = Hq // Hkv
    return h // group


def _wide(x, dtype):
    """float64 values of float32 data or of bf16 bit patterns (via torch)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float32).astype(np.float64)


@pytest.mark.parametrize("n,Hq,Hkv,dtype,t", [
    (16, 2, 2, "f32", 64), (63, 4, 2, "bf16", 64), (65, 4, 1, "f32", 64),
    (130, 8, 2, "bf16", 64), (130, 8, 2, "bf16", 1), (97, 4, 4, "f32", 8)])
def test_oracle_matches_brute(n, Hq, Hkv, dtype, t):
    p = gen.generate("tiny", 2, Hq, Hkv, n, 6, dtype, _heads(Hq), seed=n + Hq, dist="iid")
    res = O.run_layer(p.Q, p.K, p.V, dtype, p.heads, scale=0.0, slash_tile=t, workers=1)
    sc = 1 / math.sqrt(6)
    for b in range(2):
        for h in range(Hq):
            kv = _gqa(h, Hq, Hkv)
            q = _wide(p.Q[b, h], dtype).tolist()
            k = _wide(p.K[b, kv], dtype).tolist()
            v = _wide(p.V[b, kv], dtype).tolist()
            br = brute.head(q, k, v, p.heads[h].as_tuple(), sc, slash_tile=t)
            r = res["heads"][(b, h)]
            if r.kind == O.VSLASH:
                assert r.cols.tolist() == br["cols"] and r.offs.tolist() == br["offs"]
                assert np.abs(r.c - br["c"]).max() < 1e-12
                assert np.abs(r.r - br["r"]).max() < 1e-12
            if r.kind == O.BSPARSE:
                assert [x.tolist() for x in r.J] == br["J"]
            assert r.edges == br["edges"]
            o = res["O"][b, h]
            assert np.abs(o - np.array(br["o"])).max() < 1e-12
            lse = res["LSE"][b, h]
            blse = np.array(br["lse"])
            fin = np.isfinite(blse)
            assert np.array_equal(np.isfinite(lse), fin)
            assert np.abs(lse[fin] - blse[fin]).max() < 1e-12
            # per-row sets
            m = r.mask_fn(np.arange(n), n)
            for i in range(n):
                assert set(np.nonzero(m[i])[0].tolist()) == br["sets"][i]


def test_ties_in_index():
    """Identical keys make exact score ties; both implementations break them
    towards the lowest index."""
    n, dh = 70, 4
    q = np.ones((n, dh)); k = np.ones((n, dh)); v = np.arange(n * dh, dtype=float).reshape(n, dh)
    c, r = O.vs_proxy_scores(q, k, 8, 0.5)
    bc, br = brute.vs_scores(q.tolist(), k.tolist(), 8, 0.5)
    assert np.abs(c - bc).max() < 1e-12
    assert O.topk_ascending(c, 5).tolist() == brute.topk(bc, 5)
    J = O.bs_index(q, k, 1, 0, 0.5)
    assert [x.tolist() for x in J] == [[0], [0]]


def test_wrong_gqa_map_is_seen():
    """The comparison above notices a wrong GQA map: with Hq=4, Hkv=2 the
    modulo map (h % Hkv) sends head 1 to KV head 1 instead of 0, and the
    brute force over that KV head disagrees with the oracle's head 1."""
    n, Hq, Hkv, dtype = 40, 4, 2, "bf16"
    heads = [gen.ashape(2, 5), gen.ashape(2, 5), gen.ashape(2, 5), gen.ashape(2, 5)]
    p = gen.generate("tiny", 1, Hq, Hkv, n, 6, dtype, heads, seed=77, dist="iid")
    res = O.run_layer(p.Q, p.K, p.V, dtype, p.heads, workers=1)
    sc = 1 / math.sqrt(6)
    h = 1
    q = _wide(p.Q[0, h], dtype).tolist()
    right = brute.head(q, _wide(p.K[0, _gqa(h, Hq, Hkv)], dtype).tolist(),
                       _wide(p.V[0, _gqa(h, Hq, Hkv)], dtype).tolist(), heads[h].as_tuple(), sc)
    wrong = brute.head(q, _wide(p.K[0, h % Hkv], dtype).tolist(),
                       _wide(p.V[0, h % Hkv], dtype).tolist(), heads[h].as_tuple(), sc)
    assert np.abs(res["O"][0, h] - np.array(right["o"])).max() < 1e-12
    assert np.abs(res["O"][0, h] - np.array(wrong["o"])).max() > 1e-3
