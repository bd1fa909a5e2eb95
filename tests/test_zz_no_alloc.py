"""minf_sparse_attn_static, the attention entry point that allocates nothing
(its scheduler scratch is a file-scope device array of the library), against
minf_sparse_attn with a caller workspace: identical output and LSE, bit for
bit, on two calls in a row, the second with a smaller problem (the shared
scratch keeps the first call's contents)."""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from synth import gen  # noqa: E402


def _both(p):
    import torch
    prob = U.make_prob(p)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"])
    M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"],
                       buf["tiles"], buf["ws"])
    outs = []
    for static in (False, True):
        O_ = torch.full((p.B, p.Hq, p.n, p.dh), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((p.B, p.Hq, p.n), float("nan"), dtype=torch.float32, device="cuda")
        if static:
            M.minf_sparse_attn_static(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, lse)
        else:
            M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], buf["tiles"], O_, lse,
                               buf["ws"])
        torch.cuda.synchronize()
        outs.append((O_.cpu().numpy(), lse.cpu().numpy()))
    assert int(buf["tiles"]["status"].item()) == 0
    return outs


@pytest.mark.parametrize("first,second", [
    (dict(n=4100, B=2, Hq=8, Hkv=2, dh=128, seed=51), dict(n=700, B=1, Hq=4, Hkv=1, dh=128, seed=52)),
    (dict(n=2000, B=1, Hq=4, Hkv=2, dh=64, dtype="f32", dist="iid", seed=53),
     dict(n=333, B=1, Hq=2, Hkv=1, dh=64, dtype="f32", dist="iid", seed=54)),
])
def test_static_scratch_equals_workspace_path(first, second):
    for cfg in (first, second):
        U.log(f"no-alloc attention: {cfg}")
        p = gen.make_small(**cfg)
        (o_ws, l_ws), (o_st, l_st) = _both(p)
        assert np.all(np.isfinite(o_ws))
        assert np.array_equal(o_ws.view(np.uint32), o_st.view(np.uint32)), cfg
        assert np.array_equal(l_ws.view(np.uint32), l_st.view(np.uint32)), cfg
