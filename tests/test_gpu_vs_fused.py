"""GPU checks of minf_vs_index_fused, the Vertical-Slash proxy in one launch
(MInference page, section 3.1: on a GPU the index cost is counted in read
and write rounds and synchronisations; the estimate itself follows the
MInference page, section 6.2, and the blog, section 2.3.2):

* column and slash scores and the selections against the oracle, on the
  same cases as the two-launch path (several key ranges, ragged tails, GQA,
  fp32 and bf16, dh 64 and 128, n below one work-group's keys);
* scores equal the two-launch path's up to summation order;
* two runs give identical bits (fixed-order sums, no float atomics), also
  after the workspace held other data.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from oracle import minf_oracle as O  # noqa: E402
from tests.test_gpu_parity import CASES, check_index  # noqa: E402

NAMES = ["n1000_h8kv2_d128_bf16", "n333_b2_h4kv1_d64_bf16", "w1_n2048_f32_d64", "n50_h4kv4_d128_bf16",
         "n4100_h4kv1_d128_bf16_iid", "n700_h4kv2_d128_f32"]


def _run(p, fused, fill=None):
    import torch
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    if fill is not None:
        buf["ws"].fill_(fill)
    Q, K, V = U.device_inputs(p)
    c = torch.zeros((p.B, p.Hq, p.n), dtype=torch.float32, device="cuda")
    r = torch.zeros_like(c)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    if fused:
        M.minf_vs_index_fused(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"], status=st)
    else:
        M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"])
    M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
    torch.cuda.synchronize()
    assert int(st.item()) == 0, "a bounded wait of the single-launch proxy ran out"
    return buf, c.cpu().numpy(), r.cpu().numpy()


@pytest.mark.parametrize("name", NAMES)
def test_fused_proxy_matches_oracle(name):
    U.log(f"case {name}")
    p = CASES[name]()
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale)
    buf, c, r = _run(p, fused=True)
    check_index(p, res, buf, c, r)


@pytest.mark.parametrize("name", ["n1000_h8kv2_d128_bf16", "n4100_h4kv1_d128_bf16_iid", "w1_n2048_f32_d64"])
def test_fused_proxy_scores_match_two_launch_path(name):
    U.log(f"case {name}")
    p = CASES[name]()
    _, c1, r1 = _run(p, fused=True)
    _, c2, r2 = _run(p, fused=False)
    for b in range(p.B):
        for h, cfg in enumerate(p.heads):
            if cfg.kind != O.VSLASH:
                continue
            for x, y, what in ((c1, c2, "columns"), (r1, r2, "offsets")):
                scale = max(float(np.abs(y[b, h]).max()), 1e-30)
                assert np.abs(x[b, h] - y[b, h]).max() <= 1e-5 * scale, (name, b, h, what)


def test_fused_proxy_is_deterministic():
    p = CASES["n4100_h4kv1_d128_bf16_iid"]()
    b1, c1, r1 = _run(p, fused=True)
    b2, c2, r2 = _run(p, fused=True, fill=0x7f)
    assert np.array_equal(c1, c2) and np.array_equal(r1, r2)
    for k in ("vert_idx", "slash_idx"):
        assert np.array_equal(b1[k].cpu().numpy(), b2[k].cpu().numpy())


@pytest.mark.parametrize("Hkv,B", [(4, 3), (1, 2)])
def test_fused_proxy_wide_groups(Hkv, B):
    """Up to 64 VS heads in one KV group (the work order's per-group tables),
    VS heads scattered among other kinds, several batches, ragged n: against
    the oracle and the two-launch path."""
    from synth import gen
    U.log(f"wide groups Hkv={Hkv} B={B}")
    kinds = [gen.vslash(64, 30, 50), gen.vslash(20, 8, 100), gen.ashape(4, 32), gen.vslash(64, 200, 8)]
    heads = [kinds[h % 4] for h in range(64)]
    p = gen.make_small(n=700, B=B, Hq=64, Hkv=Hkv, dh=64, seed=53 + Hkv, heads=heads)
    res = O.run_layer(p.Q, p.K, p.V, p.dtype, p.heads, scale=p.scale, attend=False)
    buf, c1, r1 = _run(p, fused=True)
    check_index(p, res, buf, c1, r1)
    _, c2, r2 = _run(p, fused=False)
    for b in range(B):
        for h, cfg in enumerate(heads):
            if cfg.kind != O.VSLASH:
                continue
            for x, y in ((c1, c2), (r1, r2)):
                s = max(float(np.abs(y[b, h]).max()), 1e-30)
                assert np.abs(x[b, h] - y[b, h]).max() <= 1e-5 * s, (b, h)
