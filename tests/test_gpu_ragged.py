"""GPU checks of ragged (variable-length) batch prefill through the C ABI
(minf_prefill_ragged): the cost-model page, section 2.2 (a batch of prompts
of different lengths, no padding), with per-sample indices and no window,
slash or block crossing a sample boundary.

* every sample of a packed batch, whose attention runs in one launch over
  the work items of all samples, equals, bit for bit, the same sample run
  alone through the four calls (minf_vs_index, minf_bs_index,
  minf_build_tiles, minf_sparse_attn), kept edges included;
* changing one sample's data leaves every other sample's output unchanged;
* A-shape heads (no index estimation) match the oracle per sample;
* every pattern kind of every sample matches the oracle run on the sample's
  GPU index sets, whose selections match the oracle's estimate except
  near-ties.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from oracle import minf_oracle as O  # noqa: E402
from synth import gen  # noqa: E402


def _samples(lens, Hq, Hkv, dh, dtype, heads, seed):
    return [gen.make_small(n=n, Hq=Hq, Hkv=Hkv, dh=dh, dtype=dtype, heads=heads, seed=seed + i)
            for i, n in enumerate(lens)]


def _pack(samples):
    """Per-sample [1, H, len, dh] arrays -> the packed [H, len_b, dh] blocks
    back to back (flat)."""
    cat = lambda xs: np.concatenate([x[0].reshape(-1) for x in xs])
    return cat([s.Q for s in samples]), cat([s.K for s in samples]), cat([s.V for s in samples])


def _dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run_ragged(samples, heads_cfg, n_max, dtype):
    import torch
    s0 = samples[0]
    lens = [s.n for s in samples]
    prob = M.make_problem(len(samples), s0.Hq, s0.Hkv, n_max, s0.dh, dtype, "f32")
    heads = M.make_heads(heads_cfg)
    Qp, Kp, Vp = _pack(samples)
    T = sum(lens)
    O_ = torch.full((s0.Hq * T * s0.dh,), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((s0.Hq * T,), float("nan"), dtype=torch.float32, device="cuda")
    kept = torch.full((len(samples), s0.Hq), -1, dtype=torch.int64, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    ws = torch.empty(M.minf_ragged_ws_bytes(prob, heads, lens), dtype=torch.uint8, device="cuda")
    M.minf_prefill_ragged(prob, heads, lens, _dev(Qp, dtype), _dev(Kp, dtype), _dev(Vp, dtype), O_, lse, kept,
                          status, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    out, ls, off = [], [], 0
    O_h, lse_h = O_.cpu().numpy(), lse.cpu().numpy()
    for s in samples:
        out.append(O_h[s0.Hq * s0.dh * off: s0.Hq * s0.dh * (off + s.n)].reshape(s0.Hq, s.n, s0.dh))
        ls.append(lse_h[s0.Hq * off: s0.Hq * (off + s.n)].reshape(s0.Hq, s.n))
        off += s.n
    return out, ls, kept.cpu().numpy()


def _run_alone(s):
    import torch
    prob = U.make_prob(s, "f32")
    heads = M.make_heads(s.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(s)
    O_ = torch.full((1, s.Hq, s.n, s.dh), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((1, s.Hq, s.n), float("nan"), dtype=torch.float32, device="cuda")
    M.run_layer(prob, heads, Q, K, V, O_, lse, buf=buf)
    torch.cuda.synchronize()
    return O_[0].cpu().numpy(), lse[0].cpu().numpy(), buf["tiles"]["kept_edges"][0].cpu().numpy()


RAGGED = {
    "mixed_bf16_d128": dict(lens=[700, 1, 2113, 64, 333], Hq=8, Hkv=2, dh=128, dtype="bf16"),
    "mixed_f32_d64": dict(lens=[129, 1000, 65], Hq=4, Hkv=4, dh=64, dtype="f32"),
}


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_equals_samples_alone(name):
    c = RAGGED[name]
    base = [gen.ashape(16, 100), gen.vslash(64, 40, 60), gen.bsparse(4), gen.vslash(32, 10, 30),
            gen.bsparse(3, gen.FORCE_FIRST_BLOCK | gen.FORCE_DIAG_BLOCK), gen.ashape(0, 200), gen.vslash(64, 200, 8),
            gen.bsparse(100)]
    heads = [base[h % len(base)] for h in range(c["Hq"])]
    samples = _samples(c["lens"], c["Hq"], c["Hkv"], c["dh"], c["dtype"], heads, seed=40)
    n_max = max(c["lens"]) + 17                      # n only bounds the lengths
    out, ls, kept = _run_ragged(samples, heads, n_max, c["dtype"])
    for b, s in enumerate(samples):
        o1, l1, k1 = _run_alone(s)
        assert np.array_equal(out[b], o1), (name, b)
        assert np.array_equal(ls[b], l1), (name, b)
        assert np.array_equal(kept[b], k1), (name, b)


def test_ragged_samples_are_independent():
    import torch  # noqa: F401
    lens = [500, 300, 800]
    heads = [gen.vslash(64, 40, 60), gen.bsparse(4), gen.ashape(8, 64), gen.vslash(16, 100, 100)]
    samples = _samples(lens, 4, 2, 128, "bf16", heads, seed=70)
    out_a, _, kept_a = _run_ragged(samples, heads, 800, "bf16")
    other = _samples([300], 4, 2, 128, "bf16", heads, seed=99)[0]
    changed = [samples[0], other, samples[2]]
    out_b, _, kept_b = _run_ragged(changed, heads, 800, "bf16")
    for b in (0, 2):
        assert np.array_equal(out_a[b], out_b[b]) and np.array_equal(kept_a[b], kept_b[b]), b
    assert not np.array_equal(out_a[1], out_b[1])


def test_ragged_ashape_matches_oracle():
    lens = [257, 64, 1000]
    heads = [gen.ashape(16, 100), gen.ashape(0, 64), gen.ashape(64, 0), gen.ashape(3, 500)]
    samples = _samples(lens, 4, 2, 128, "bf16", heads, seed=5)
    out, ls, kept = _run_ragged(samples, heads, 1000, "bf16")
    for b, s in enumerate(samples):
        ref = O.run_layer(s.Q, s.K, s.V, s.dtype, s.heads)
        U.compare_output(out[b][None], ref["O"], s.dtype, f"ragged sample {b}")
        for h, cfg in enumerate(heads):
            assert kept[b, h] == O.ashape_row_counts(s.n, cfg.sink, cfg.window).sum()


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_matches_oracle_all_kinds(name):
    """Every pattern kind of every packed sample against the oracle.  A
    packed sample's index sets stay inside the workspace, so they are taken
    from the same sample run alone, which the packed run equals bit for bit
    (checked here again): those selections must match the oracle's estimate
    except near-ties, and the packed output rows and kept edges must match
    the oracle's attention over them."""
    c = RAGGED[name]
    base = [gen.vslash(64, 40, 60), gen.bsparse(4), gen.ashape(16, 100), gen.vslash(32, 10, 30),
            gen.bsparse(3, gen.FORCE_FIRST_BLOCK | gen.FORCE_DIAG_BLOCK), gen.ashape(0, 200), gen.vslash(64, 200, 8),
            gen.bsparse(100)]
    heads = [base[h % len(base)] for h in range(c["Hq"])]
    samples = _samples(c["lens"], c["Hq"], c["Hkv"], c["dh"], c["dtype"], heads, seed=140)
    out, ls, kept = _run_ragged(samples, heads, max(c["lens"]), c["dtype"])
    import torch
    for b, s in enumerate(samples):
        prob = U.make_prob(s, "f32")
        hh = M.make_heads(s.heads)
        buf = M.alloc_buffers(prob, hh)
        Q, K, V = U.device_inputs(s)
        O1 = torch.zeros((1, s.Hq, s.n, s.dh), dtype=torch.float32, device="cuda")
        M.run_layer(prob, hh, Q, K, V, O1, buf=buf)
        torch.cuda.synchronize()
        assert np.array_equal(out[b], O1[0].cpu().numpy()), (name, b)
        est = O.run_layer(s.Q, s.K, s.V, s.dtype, s.heads, scale=s.scale, attend=False)
        given = U.gpu_given(s, buf)
        for (bb, h), r in est["heads"].items():
            cfg = s.heads[h]
            if r.kind == O.VSLASH:
                cols, offs = given[(bb, h)]
                U.check_selection(cols, r.c, cfg.n_vertical, f"sample {b} head {h} columns")
                U.check_selection(offs, r.r, cfg.n_slash, f"sample {b} head {h} offsets")
            elif r.kind == O.BSPARSE:
                sc = O.bs_block_scores(O.widen(s.Q[0, h], s.dtype),
                                       O.widen(s.K[0, O.kv_head(h, s.Hq, s.Hkv)], s.dtype), s.eff_scale)
                J = given[(bb, h)]
                Jm = np.full((len(J), max(1, max(len(x) for x in J))), -1, dtype=np.int64)
                for u, x in enumerate(J):
                    Jm[u, :len(x)] = x
                U.check_block_selections(Jm, [len(x) for x in J], sc, cfg.topk_blocks, cfg.force_flags,
                                         f"sample {b} head {h}")
        ref = O.run_layer(s.Q, s.K, s.V, s.dtype, s.heads, scale=s.scale, given=given)
        U.compare_output(out[b][None], ref["O"], s.dtype, f"{name} packed sample {b} (n={s.n})")
        for h in range(s.Hq):
            assert kept[b, h] == ref["heads"][(0, h)].edges, (name, b, h)
