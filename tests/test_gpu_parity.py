"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Level 1: the oracle's index sets are fed to minf_build_tiles and
minf_sparse_attn; tile lists and kept edges must match exactly and the
output element by element (bf16 inputs: max-abs 1e-2 and mean-abs 1e-3;
fp32 inputs: 1e-5).  Level 2: minf_vs_index / minf_bs_index must select the
oracle's sets except for near-ties (oracle score within 1e-4 relative of the
k-th threshold).  End to end: the whole path's output and kept edges match
the oracle's attention over the GPU's own index sets.
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


def _small_cases():
    return {
        "w1_n2048_f32_d64": lambda: gen.make_workload(1),
        "n1000_h8kv2_d128_bf16": lambda: gen.make_small(n=1000, Hq=8, Hkv=2, dh=128),
        "n333_b2_h4kv1_d64_bf16": lambda: gen.make_small(n=333, B=2, Hq=4, Hkv=1, dh=64, seed=3),
        "n50_h4kv4_d128_bf16": lambda: gen.make_small(n=50, Hq=4, Hkv=4, dh=128, seed=5),
        "n1_h2kv1_d64_f32": lambda: gen.make_small(n=1, Hq=2, Hkv=1, dh=64, dtype="f32", dist="iid", seed=9),
        "n700_h4kv2_d128_f32": lambda: gen.make_small(n=700, Hq=4, Hkv=2, dh=128, dtype="f32", dist="iid", seed=11),
        "n4100_h4kv1_d128_bf16_iid": lambda: gen.make_small(
            n=4100, Hq=4, Hkv=1, dh=128, dist="iid", seed=13,
            heads=[gen.vslash(64, 0, 3), gen.ashape(0, 1), gen.bsparse(1), gen.vslash(17, 5, 0)]),
    }


CASES = _small_cases()


def _run_attn_given(p, res, out_dtype="f32", slash_tile=64):
    import torch
    prob = U.make_prob(p, out_dtype)
    prob.slash_tile = slash_tile
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    U.load_oracle_indices(p, res, buf)
    Q, K, V = U.device_inputs(p)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    O_ = torch.full((p.B, p.Hq, p.n, p.dh), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((p.B, p.Hq, p.n), float("nan"), dtype=torch.float32, device="cuda")
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"],
                       buf["tiles"], buf["ws"])
    M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, lse, buf["ws"])
    torch.cuda.synchronize()
    return buf, O_.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_attention_given_oracle_indices(name):
    U.log(f"case {name}")
    p = CASES[name]()
    with U.Timer("oracle"):
        res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale)
    with U.Timer("gpu"):
        buf, Og, lse = _run_attn_given(p, res)
    U.check_tiles(p, res, buf)
    U.compare_output(Og, res["O"], p.dtype, f"{name} O")
    fin = np.isfinite(res["LSE"])
    assert np.array_equal(np.isfinite(lse), fin), "empty rows differ"
    assert np.abs(lse[fin] - res["LSE"][fin]).max(initial=0.0) < (2e-2 if p.dtype == "bf16" else 1e-5)
    # empty rows are exactly zero
    assert np.all(Og[~fin] == 0)


def test_bf16_output_dtype():
    p = CASES["n1000_h8kv2_d128_bf16"]()
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads)
    _, Og, _ = _run_attn_given(p, res, out_dtype="bf16")
    # a bf16 output adds its own rounding (2^-9 relative): compare with that allowance
    d = np.abs(Og - res["O"]) - np.abs(res["O"]) * 2.0 ** -8
    assert d.max() <= U.BF16_MAX_ABS


def _run_index(p):
    import torch
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    c = torch.zeros((p.B, p.Hq, p.n), dtype=torch.float32, device="cuda")
    r = torch.zeros_like(c)
    M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"])
    M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
    torch.cuda.synchronize()
    return prob, heads, buf, (Q, K, V), c.cpu().numpy(), r.cpu().numpy()


def check_index(p, res, buf, c, r):
    """Selections and proxy scores against the oracle; returns True when the
    GPU sets equal the oracle's exactly."""
    vi = buf["vert_idx"].cpu().numpy()
    si = buf["slash_idx"].cpu().numpy()
    bi = buf["blk_idx"].cpu().numpy()
    bc = buf["blk_cnt"].cpu().numpy()
    exact = True
    ndiff = nex = 0
    for (b, h), hr in res["heads"].items():
        cfg = p.heads[h]
        if hr.kind == O.VSLASH:
            # proxy scores: fp32 sums of probabilities vs fp64
            sc = max(hr.c.max(), 1e-30)
            assert np.abs(c[b, h] - hr.c).max() <= 2e-5 * sc + 1e-7, "column scores"
            sr = max(hr.r.max(), 1e-30)
            assert np.abs(r[b, h] - hr.r).max() <= 2e-5 * sr + 1e-7, "diagonal scores"
            d1, e1 = U.check_selection(vi[b, h], hr.c, cfg.n_vertical, f"columns ({b},{h})")
            d2, e2 = U.check_selection(si[b, h], hr.r, cfg.n_slash, f"offsets ({b},{h})")
            ndiff += d1 + d2
            nex += e1 + e2
        elif hr.kind == O.BSPARSE:
            scores = O.bs_block_scores(O.widen(p.Q[b, h], p.dtype), O.widen(p.K[b, O.kv_head(h, p.Hq, p.Hkv)], p.dtype),
                                       p.eff_scale)
            for u, J in enumerate(hr.J):
                row = scores[u, :u + 1].copy()
                if cfg.force_flags & O.FORCE_FIRST_BLOCK:
                    row[0] = np.inf
                if cfg.force_flags & O.FORCE_DIAG_BLOCK:
                    row[u] = np.inf
                assert bc[b, h, u] == len(J)
                d, e = U.check_selection(bi[b, h, u, :bc[b, h, u]], row, cfg.topk_blocks, f"blocks ({b},{h},{u})")
                ndiff += d
                nex += e
    U.log(f"  index: {ndiff} differing selections, {nex} exempt near-ties")
    return ndiff == 0


@pytest.mark.parametrize("name", ["n1000_h8kv2_d128_bf16", "n333_b2_h4kv1_d64_bf16", "w1_n2048_f32_d64",
                                  "n50_h4kv4_d128_bf16", "n4100_h4kv1_d128_bf16_iid", "n700_h4kv2_d128_f32"])
def test_index_and_end_to_end(name):
    import torch
    U.log(f"case {name}")
    p = CASES[name]()
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale)
    prob, heads, buf, (Q, K, V), c, r = _run_index(p)
    exact = check_index(p, res, buf, c, r)
    # end to end on the GPU's own indices
    O_ = torch.zeros((p.B, p.Hq, p.n, p.dh), dtype=torch.float32, device="cuda")
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"],
                       buf["tiles"], buf["ws"])
    M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, None, buf["ws"])
    torch.cuda.synchronize()
    assert int(buf["tiles"]["status"].item()) == 0
    # the oracle's attention on the GPU's own index sets (the same sets as
    # the oracle's estimate unless a near-tie differs)
    U.log(f"  GPU index sets identical to the oracle's: {exact}")
    ref = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale, given=U.gpu_given(p, buf))
    U.compare_output(O_.cpu().numpy(), ref["O"], p.dtype, f"{name} end-to-end O")
    ke = buf["tiles"]["kept_edges"].cpu().numpy()
    for (b, h), hr in ref["heads"].items():
        assert int(ke[b, h]) == hr.edges


def test_determinism():
    """No floating-point atomics: two runs of the whole path are bit-identical."""
    import torch
    p = CASES["n1000_h8kv2_d128_bf16"]()
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    Q, K, V = U.device_inputs(p)
    outs = []
    for _ in range(2):
        O_ = torch.zeros((p.B, p.Hq, p.n, p.dh), dtype=torch.float32, device="cuda")
        buf = M.run_layer(prob, heads, Q, K, V, O_)
        torch.cuda.synchronize()
        outs.append((O_.cpu().numpy(), buf["vert_idx"].cpu().numpy(), buf["slash_idx"].cpu().numpy(),
                     buf["blk_idx"].cpu().numpy(), buf["tiles"]["kept_edges"].cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_bad_indices_set_status_and_stay_in_bounds():
    """Malformed indices written by the host: the tile builder flags them in
    the status word, and attention keeps nothing for those heads instead of
    reading outside K/V."""
    import torch
    p = gen.make_small(n=500, Hq=4, Hkv=2, dh=128, seed=21,
                       heads=[gen.vslash(64, 8, 8), gen.bsparse(2), gen.vslash(64, 8, 8), gen.ashape(4, 16)])
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    vi = torch.arange(8, dtype=torch.int32).repeat(1, 4, 1).cuda()
    si = torch.tensor([5, 3, 9, 10, 11, 12, 13, 14], dtype=torch.int32).repeat(1, 4, 1).cuda()   # not ascending
    buf["vert_idx"][..., :8] = vi
    buf["slash_idx"][..., :8] = si
    buf["blk_idx"].fill_(1000)                      # beyond every causal block
    buf["blk_cnt"].fill_(2)
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"],
                       buf["tiles"], buf["ws"])
    O_ = torch.zeros((1, 4, 500, 128), dtype=torch.float32, device="cuda")
    M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, None, buf["ws"])
    torch.cuda.synchronize()
    st = int(buf["tiles"]["status"].item())
    assert st & M.MINF_DEV_BAD_SLASH and st & M.MINF_DEV_BAD_BLOCK
    o = O_.cpu().numpy()
    assert np.all(o[0, 0] == 0) and np.all(o[0, 1] == 0) and np.all(o[0, 2] == 0)
    assert np.all(np.isfinite(o[0, 3])) and np.abs(o[0, 3]).max() > 0


@pytest.mark.parametrize("n", [1000, 2113])
def test_dense_causal_baseline_as_full_window(n):
    """The dense causal baseline runs on the same kernels as an A-shape head
    with no sink and a window of n keys, i.e. N(i) = {j <= i} ([MInf]
    section 1.1, Eq. 1-2).  Checked against the textbook dense causal
    softmax attention of the oracle, and kept edges = n(n+1)/2 per head."""
    U.log(f"dense n={n}")
    p = gen.make_small(n=n, Hq=4, Hkv=2, dh=128, seed=21, heads=[gen.ashape(0, n)] * 4)
    import torch
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    O_ = torch.full((p.B, p.Hq, n, p.dh), float("nan"), dtype=torch.float32, device="cuda")
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"],
                       buf["tiles"], buf["ws"])
    M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, None, buf["ws"])
    torch.cuda.synchronize()
    ke = buf["tiles"]["kept_edges"].cpu().numpy()
    assert np.all(ke == n * (n + 1) // 2)
    Og = O_.cpu().numpy()
    ref = np.zeros_like(Og, dtype=np.float64)
    g = p.Hq // p.Hkv
    for h in range(p.Hq):
        q = O.widen(p.Q[0, h], p.dtype)
        k = O.widen(p.K[0, h // g], p.dtype)
        v = O.widen(p.V[0, h // g], p.dtype)
        ref[0, h], _ = O.dense_attention(q, k, v, p.eff_scale)
    U.compare_output(Og, ref, p.dtype, f"dense n={n}")


EXACT_CASES = ["n1000_h8kv2_d128_bf16", "n333_b2_h4kv1_d64_bf16", "n700_h4kv2_d128_f32", "n4100_h4kv1_d128_bf16_iid"]


@pytest.mark.parametrize("name", EXACT_CASES)
def test_exact_slash_pairs_given_oracle_indices(name):
    """slash_tile=1: Eq. 5 taken literally (row i keeps key j iff i - j is a
    selected offset or j a selected column, j <= i).  Same tile lists; kept
    edges and every output row against the oracle run with slash_tile=1."""
    U.log(f"exact case {name}")
    p = CASES[name]()
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale, slash_tile=1)
    buf, Og, lse = _run_attn_given(p, res, slash_tile=1)
    U.check_tiles(p, res, buf)
    U.compare_output(Og, res["O"], p.dtype, f"{name} O (exact pairs)")
    fin = np.isfinite(res["LSE"])
    assert np.array_equal(np.isfinite(lse), fin), "empty rows differ"
    assert np.abs(lse[fin] - res["LSE"][fin]).max(initial=0.0) < (2e-2 if p.dtype == "bf16" else 1e-5)
    assert np.all(Og[~fin] == 0)


def test_many_batch_heads():
    """More (batch, head) pairs than the attention scheduler stages in LDS
    (B * Hq = 4160 > 4096 units): the schedule falls back to global memory;
    every kind, ragged n, against the oracle."""
    U.log("many batch x heads")
    base = [gen.ashape(16, 40), gen.vslash(32, 8, 16), gen.bsparse(2), gen.vslash(16, 4, 4)]
    p = gen.make_small(n=150, B=65, Hq=64, Hkv=16, dh=128, seed=31, heads=[base[h % 4] for h in range(64)])
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale)
    buf, Og, lse = _run_attn_given(p, res)
    U.check_tiles(p, res, buf)
    U.compare_output(Og, res["O"], p.dtype, "B=65 Hq=64 O")
