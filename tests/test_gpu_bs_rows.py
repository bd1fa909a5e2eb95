"""Block-Sparse row top-k on long rows with designed block scores (GPU).

Every query row is e_0 and every key row of block j is f(j) e_0, so the
pooled score of query block u against key block j is scale * f(j) exactly
(PaperTrace 2.1.2 "MInference", section 2, Eq. 6: mean-pooled queries and
keys, one score per causal block pair).  The expected block list of each row
is then the selection rule written out: the k highest scores among blocks
0..u, ties to the lowest block, the forced first and diagonal blocks taking
slots inside the budget; no oracle run is needed.

The rows reach 4608 blocks, so they cover every kernel width of the row
selection, including the rows (2048 blocks and more) whose candidates are
first bounded by a sample of the row (one score per thread).  The patterns
drive each outcome of that bound:
* high scores exactly at the sampled positions: the sample's threshold keeps
  fewer than k blocks, and the selection falls back to the whole row;
* high scores on every fifth block: the threshold keeps a few hundred blocks,
  all tied, and the selection runs on the candidates alone, where the ties
  must still go to the lowest blocks;
* all scores equal: every block passes the threshold, more than the
  candidate space holds, and the selection falls back again.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

NQ = 4608           # query and key blocks
N = 64 * NQ
DH = 128
K_BLOCKS = 256
FORCE_FIRST, FORCE_DIAG = 1, 2


def _patterns():
    j = np.arange(NQ)
    return {
        # 3 on the blocks every row's sample reads (multiples of 32 cover the
        # sampled positions of both the 16- and 32-wide rows), 2 on the other
        # multiples of 16, 1 elsewhere
        "sampled_high": np.where(j % 32 == 0, 3.0, np.where(j % 16 == 0, 2.0, 1.0)),
        "every_fifth": np.where(j % 5 == 0, 2.0, 1.0),
        "all_equal": np.ones(NQ),
    }


def _expected(f, u, k, force):
    """The selection rule on row u: blocks 0..u by score descending, then
    block ascending; forced blocks rank above every score."""
    s = f[: u + 1].copy()
    if force & FORCE_FIRST:
        s[0] = np.inf
    if force & FORCE_DIAG:
        s[u] = np.inf
    order = np.lexsort((np.arange(u + 1), -s))
    return np.sort(order[: min(k, u + 1)])


@pytest.mark.parametrize("force", [0, FORCE_FIRST | FORCE_DIAG])
@pytest.mark.parametrize("pattern", ["sampled_high", "every_fifth", "all_equal"])
def test_long_rows_designed_scores(pattern, force):
    import torch

    import long_context_prefill_amd as M
    from synth import gen

    f = _patterns()[pattern]
    print(f"Block-Sparse rows: pattern {pattern}, force {force}, {NQ} blocks", flush=True)
    # bf16 bits of 1.0, 2.0 and 3.0 are exact; rows of one block are equal,
    # so the 64-row means are exact too
    Qrow = np.zeros(DH)
    Qrow[0] = 1.0
    Q = np.broadcast_to(gen.f64_to_bf16_bits(Qrow), (1, 1, N, DH))
    kvals = gen.f64_to_bf16_bits(np.repeat(f, 64)[:, None] * np.eye(1, DH))
    K = kvals.reshape(1, 1, N, DH)
    conv = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    Qd, Kd = conv(Q), conv(K)
    prob = M.make_problem(1, 1, 1, N, DH, "bf16", "f32")
    heads = M.make_heads([gen.bsparse(K_BLOCKS, force)])
    buf = M.alloc_buffers(prob, heads)
    M.minf_bs_index(prob, heads, Qd, Kd, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
    torch.cuda.synchronize()
    idx = buf["blk_idx"][0, 0].cpu().numpy()
    cnt = buf["blk_cnt"][0, 0].cpu().numpy()
    bad = []
    for u in range(NQ):
        want = _expected(f, u, K_BLOCKS, force)
        got = idx[u, : cnt[u]]
        if cnt[u] != len(want) or not np.array_equal(got, want) or np.any(idx[u, cnt[u]:] != -1):
            bad.append(u)
    print(f"  {NQ - len(bad)}/{NQ} rows match the closed form", flush=True)
    assert not bad, f"rows differing: {bad[:10]} (of {len(bad)})"
