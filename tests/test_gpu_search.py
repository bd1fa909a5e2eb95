"""GPU checks of the offline pattern search (PaperTrace 2.1.2 "MInference",
sections 3.1 and 6.3; blog-zz7 "LLM模型之MInference", section 2.3.1, Eq. 2)
through the C ABI: minf_output_error against the oracle's definition, and the
search's per-head error table on small calibration layers against the
oracle's (each candidate's output from the oracle's own index estimation and
restricted softmax, against the oracle's dense attention)."""
import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from long_context_prefill_amd import search as S  # noqa: E402
from oracle import minf_oracle as O  # noqa: E402
from synth import gen  # noqa: E402


def _dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("B,Hq,n,dh,out", [(2, 3, 77, 64, "f32"), (1, 4, 1000, 128, "bf16"), (1, 1, 1, 64, "f32")])
def test_output_error_matches_oracle(B, Hq, n, dh, out):
    import torch
    rng = np.random.default_rng(B * 100 + n)
    a = rng.standard_normal((B, Hq, n, dh))
    r = a + 0.1 * rng.standard_normal((B, Hq, n, dh))
    r[:, 0] = a[:, 0]                                    # a head with no error
    if out == "bf16":
        ab, rb = gen.f64_to_bf16_bits(a), gen.f64_to_bf16_bits(r)
        av, rv = gen.bf16_bits_to_f32(ab), gen.bf16_bits_to_f32(rb)
        A, R = _dev(ab, "bf16"), _dev(rb, "bf16")
    else:
        av, rv = a.astype(np.float32), r.astype(np.float32)
        A, R = _dev(av, "f32"), _dev(rv, "f32")
    prob = M.make_problem(B, Hq, 1, n, dh, "f32", out)
    err = torch.empty(2 * B * Hq, dtype=torch.float64, device="cuda")
    M.minf_output_error(prob, A, R, err)
    first = err.cpu().numpy().copy()
    M.minf_output_error(prob, A, R, err)
    assert np.array_equal(first, err.cpu().numpy())         # fixed order: identical bits
    got = first.reshape(B, Hq, 2)
    for b in range(B):
        d2, r2 = O.output_error(av[b:b + 1], rv[b:b + 1])
        assert np.allclose(got[b, :, 0], d2, rtol=1e-12, atol=0), (b, got[b, :, 0], d2)
        assert np.allclose(got[b, :, 1], r2, rtol=1e-12, atol=0)
        assert got[b, 0, 0] == 0.0


@pytest.mark.parametrize("B,Hq,n", [(2, 3, 77), (1, 4, 1000), (1, 1, 1)])
def test_captured_mass_matches_definition(B, Hq, n):
    import torch
    rng = np.random.default_rng(7 * n + Hq)
    ref = rng.standard_normal((B, Hq, n)).astype(np.float32) + 5.0
    lse = (ref - rng.uniform(0.0, 3.0, size=ref.shape)).astype(np.float32)
    lse.reshape(-1)[::5] = -np.inf                       # rows without a kept key add 0
    prob = M.make_problem(B, Hq, 1, n, 64, "f32", "f32")
    mass = torch.empty(B * Hq, dtype=torch.float64, device="cuda")
    M.minf_captured_mass(prob, torch.from_numpy(lse).cuda(), torch.from_numpy(ref).cuda(), mass)
    got = mass.cpu().numpy().reshape(B, Hq)
    want = np.exp(lse.astype(np.float64) - ref.astype(np.float64)).sum(axis=2)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


SEARCH_CASES = {
    "n1024_h6kv3_d64_f32": dict(n=1024, Hq=6, Hkv=3, dh=64, dtype="f32", tol=(1e-4, 1e-3), mtol=1e-4),
    "n1024_h6kv3_d128_bf16": dict(n=1024, Hq=6, Hkv=3, dh=128, dtype="bf16", tol=(4e-3, 0.03), mtol=2e-3),
}


@pytest.mark.parametrize("name", list(SEARCH_CASES))
def test_pattern_search_matches_oracle(name):
    c = SEARCH_CASES[name]
    n, Hq, Hkv, dh, dt = c["n"], c["Hq"], c["Hkv"], c["dh"], c["dtype"]
    p = gen.make_calibration(n=n, Hq=Hq, Hkv=Hkv, dh=dh, dtype=dt, period=128, harmonics=8, n_sinks=4,
                             n_clusters=8)
    grid = [S.ashape(16, 128), S.ashape(32, 512), S.vslash(64, 64, 128), S.vslash(64, 128, 256),
            S.bsparse(2), S.bsparse(4), S.dense(n)]
    eps = 0.05
    prob = M.make_problem(1, Hq, Hkv, n, dh, dt, "f32")
    res = S.search(prob, _dev(p.Q, dt), _dev(p.K, dt), _dev(p.V, dt), grid=grid, eps=eps, reps=2)
    print(name, "times", [round(t, 3) for t in res["times_ms"]], "choice", res["choice"], flush=True)

    dense = O.run_layer(p.Q, p.K, p.V, dt, [gen.HeadCfg(*S.dense(n))] * Hq)["O"]
    atol, rtol = c["tol"]
    for ci, cfg in enumerate(grid):
        heads = [gen.HeadCfg(*cfg)] * Hq
        out = O.run_layer(p.Q, p.K, p.V, dt, heads)["O"]
        want = O.relative_output_error(out, dense)
        got = np.array([res["rel_err"][h][ci] for h in range(Hq)])
        assert np.all(np.abs(got - want) <= atol + rtol * want), (S.describe(cfg), got, want)
        # missed attention mass: the GPU's lse route against the oracle's
        # explicit probabilities
        want_m = O.layer_missed_mass(p.Q, p.K, dt, heads)
        got_m = np.array([res["missed_mass"][h][ci] for h in range(Hq)])
        assert np.all(np.abs(got_m - want_m) <= c["mtol"]), (S.describe(cfg), got_m, want_m)

    # the dense candidate reproduces the dense run exactly
    assert all(res["rel_err"][h][-1] == 0.0 and res["missed_mass"][h][-1] == 0.0 for h in range(Hq))
    # the choice is the oracle's rule applied to the measured table
    assert res["measure"] == "mass"
    assert res["choice"] == O.choose_patterns(res["missed_mass"], res["times_ms"], eps)
    # every chosen head is within the bound, and running the chosen table
    # reproduces each head's candidate errors exactly (heads are independent)
    for h in range(Hq):
        ch = res["choice"][h]
        assert res["missed_mass"][h][ch] <= eps
        assert res["table_missed_mass"][h] == res["missed_mass"][h][ch]
        assert res["table_rel_err"][h] == res["rel_err"][h][ch]
    # no candidate within the bound is faster than the chosen one
    for h in range(Hq):
        ch = res["choice"][h]
        for ci in range(len(grid)):
            if res["missed_mass"][h][ci] <= eps:
                assert res["times_ms"][ci] >= res["times_ms"][ch]
