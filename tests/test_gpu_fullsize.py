"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (whole layer: Vertical-Slash index,
Block-Sparse index, tile build, sparse attention, fp32 output).

For every workload and EVERY head:
* its index against the oracle's: Vertical-Slash columns and offsets, and
  every query block's Block-Sparse selection, identical except candidates
  whose oracle score lies within 1e-4 relative of the k-th threshold;
* its kept edges, exactly, against the oracle's count over the GPU's own
  index sets;
* its output rows against the oracle's restricted softmax over the GPU's own
  index sets (max-abs 1e-2, mean-abs 1e-3 for bf16 inputs): all rows up to
  32K tokens; above that the 4096 seeded sampled rows plus the edge rows
  {0, 1, 63, 64, 65, n/2, n-65, n-64, n-1}.
The oracle runs on a pool of threads, one KV group at a time (its four
query heads share the widened K and V), each head's rows split over
several tasks.  Every row of a sequence up to 32K tokens is checked with
masked dense products of row chunks (O.attend_rows); the sampled rows of the
longer sequences row by row over their candidate key ranges
(O.attend_rows_ranges, plain C in double precision), which costs what the
row keeps rather than the whole prefix.
"""
import math
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from tests.conftest import gpu_available
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from oracle import minf_oracle as O  # noqa: E402
from synth import gen  # noqa: E402


def _threads():
    try:
        c = len(os.sched_getaffinity(0))
    except AttributeError:
        c = os.cpu_count() or 1
    return max(1, min(16, c))


def _f32(x, dtype):
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _row_refs(q, k, v, rows, keys_fn, scale, what):
    """Oracle rows (float64 arithmetic on exactly widened inputs), on threads."""

    def one(i):
        keys = keys_fn(int(i))
        return O.attend_row_keys(q[i].astype(np.float64), k, v, keys, scale)

    out = np.zeros((len(rows), v.shape[1]))
    t0 = time.time()
    with ThreadPoolExecutor(_threads()) as ex:
        for t, (o, _) in enumerate(ex.map(one, rows)):
            out[t] = o
            if t % 512 == 511:
                U.log(f"    {what}: {t + 1}/{len(rows)} oracle rows ({time.time() - t0:.0f}s)")
    return out


class _Widened:
    """float64 view of fp32 rows, built on demand (k[keys] -> float64)."""

    def __init__(self, a32):
        self.a = a32

    def __getitem__(self, idx):
        return self.a[idx].astype(np.float64)

    @property
    def shape(self):
        return self.a.shape


def _check_index(p, given, cnt, h, k64):
    """Head h's GPU selections against the oracle's estimate (k64: its KV
    head's keys in float64); returns the number of (exempt) differences."""
    cfg = p.heads[h]
    q = _Widened(_f32(p.Q[0, h], p.dtype))
    if cfg.kind == gen.VSLASH:
        c, r = O.vs_proxy_scores(q, k64, cfg.last_q, p.eff_scale)
        cols, offs = given[(0, h)]
        d1, _ = U.check_selection(cols, c, cfg.n_vertical, f"head {h} columns")
        d2, _ = U.check_selection(offs, r, cfg.n_slash, f"head {h} offsets")
        return d1 + d2
    if cfg.kind == gen.BSPARSE:
        scores = O.bs_block_scores(q, k64, p.eff_scale)
        J = given[(0, h)]
        Jm = np.full((len(J), max(1, max(len(x) for x in J))), -1, dtype=np.int64)
        for u, x in enumerate(J):
            Jm[u, :len(x)] = x
        return U.check_block_selections(Jm, cnt[0, h], scores, cfg.topk_blocks, cfg.force_flags, f"head {h}")[0]
    return 0


def _check_group(p, kv, rows, given, cnt, ke, ref, nt):
    """KV group kv's query heads: each head's index against the oracle's
    estimate, its kept edges (ke) against the oracle's count over the GPU's
    index sets (given, cnt), and the oracle's output rows over those sets
    into ref[h].  Returns the number of exempt near-tie differences."""
    from threadpoolctl import threadpool_limits
    n, g, sc = p.n, p.Hq // p.Hkv, p.eff_scale
    parts = max(1, nt // g)
    k64 = O.widen(p.K[0, kv], p.dtype)
    hs = list(range(kv * g, (kv + 1) * g))
    res = {h: O.head_index(None, None, p.heads[h], n, sc, 64, O.BLOCK, given.get((0, h))) for h in hs}
    sampled = p.rows is not None
    if sampled:
        # sampled rows of a long sequence: row by row over the listed key
        # ranges, in C (a row keeps a small share of the keys before it)
        k32, v32 = _f32(p.K[0, kv], p.dtype), _f32(p.V[0, kv], p.dtype)
        fns = {}
        for h in hs:
            cfg, r = p.heads[h], res[h]
            if r.kind == O.ASHAPE:
                fns[h] = lambda i, cfg=cfg: O.ashape_row_ranges(i, cfg.sink, cfg.window)
            elif r.kind == O.BSPARSE:
                fns[h] = lambda i, r=r: O.bs_row_ranges(i, r.J)
            else:
                cover = O.slash_offset_set(r.offs, n, 64)
                runs = O.span_runs(cover, 64)
                fns[h] = lambda i, r=r, cover=cover, runs=runs: O.vs_row_ranges(i, r.cols, cover, 64, runs)
    else:
        v64 = O.widen(p.V[0, kv], p.dtype)

    def job(j):
        if j[0] == "index":
            return j, _check_index(p, given, cnt, j[1], k64)
        if j[0] == "edges":
            return j, res[j[1]].edges
        h, part = j[1], j[2]
        rr = rows[part::parts]
        if sampled:
            o, _ = O.attend_rows_ranges(_f32(p.Q[0, h][rr], p.dtype), k32, v32, rr, fns[h], sc)
        else:
            # every row: dense products of row chunks against the keys up to
            # the chunk's last row, masked
            o, _ = O.attend_rows(_Widened(_f32(p.Q[0, h], p.dtype)), k64, v64, rr, res[h].mask_fn, sc)
        return j, o

    jobs = ([("attn", h, part) for h in hs for part in range(parts)] + [("index", h) for h in hs] +
            [("edges", h) for h in hs])
    ndiff = 0
    with threadpool_limits(limits=1), ThreadPoolExecutor(nt) as ex:
        for j, r in ex.map(job, jobs):
            if j[0] == "attn":
                ref[j[1], j[2]::parts] = r
            elif j[0] == "index":
                ndiff += r
            else:
                assert int(ke[0, j[1]]) == r, f"kept edges of head {j[1]}: {ke[0, j[1]]} vs {r}"
    return ndiff


@pytest.mark.timeout(700)
@pytest.mark.parametrize("w", [2, 3, 4, 5])
def test_full_size_layer(w):
    import torch
    t0 = time.time()
    p = gen.make_workload(w)
    U.log(f"workload {p.name}: generated in {time.time() - t0:.0f}s")
    n = p.n
    g = p.Hq // p.Hkv
    sc = p.eff_scale
    prob = M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, "f32", p.scale)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    Og = torch.empty((p.B, p.Hq, n, p.dh), dtype=torch.float32, device="cuda")
    t = buf["tiles"]
    M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"])
    M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
    M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"], t, buf["ws"])
    M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], t, Og, None, buf["ws"])
    torch.cuda.synchronize()
    assert int(t["status"].item()) == 0
    U.log(f"  GPU layer done ({time.time() - t0:.0f}s)")
    if p.rows is None:
        rows = np.arange(n, dtype=np.int64)
    else:
        rows = np.unique(np.concatenate([p.rows, p.edge_rows])).astype(np.int64)
    given = U.gpu_given(p, buf)
    cnt = buf["blk_cnt"].cpu().numpy()
    ke = t["kept_edges"].cpu().numpy()
    og = Og[0][:, torch.from_numpy(rows).cuda()].cpu().numpy()          # [Hq, R, dh]
    del Q, K, V, Og, buf, t
    torch.cuda.empty_cache()
    nt = _threads()

    # ---- per KV group (its query heads share the widened K and V): every
    #      head's index against the oracle's estimate, its kept edges and its
    #      output rows against the oracle's attention on the GPU's index sets
    ref = np.zeros((p.Hq, len(rows), p.dh))
    ndiff = 0
    for kv in range(p.Hkv):
        hs = list(range(kv * g, (kv + 1) * g))
        ndiff += _check_group(p, kv, rows, given, cnt, ke, ref, nt)
        U.log(f"  KV group {kv}: heads {hs[0]}..{hs[-1]} ({', '.join(gen.KIND_NAMES[p.heads[h].kind] for h in hs)}): "
              f"index, kept edges and oracle rows done ({time.time() - t0:.0f}s)")
    U.log(f"  index of all {p.Hq} heads matches the oracle's ({ndiff} near-tie differences)")
    worst = (0.0, 0.0)
    for h in range(p.Hq):
        mx, mean = U.compare_output(og[h], ref[h], p.dtype,
                                    f"{p.name} head {h} ({gen.KIND_NAMES[p.heads[h].kind]}), {len(rows)} rows")
        worst = (max(worst[0], mx), max(worst[1], mean))
    U.log(f"  {p.name}: {p.Hq}/{p.Hq} heads x {len(rows)} rows match; worst max-abs {worst[0]:.3e}, "
          f"worst mean-abs {worst[1]:.3e} ({time.time() - t0:.0f}s)")


@pytest.mark.timeout(400)
def test_full_size_exact_slash_pairs():
    """The 128K mixed layer with slash_tile=1 (Eq. 5 pairs): one
    Vertical-Slash head's kept edges against the oracle's count over the
    GPU's own index sets, and its 4096 sampled + edge rows against the
    oracle's restricted softmax over the exact-pair key sets."""
    import torch
    t0 = time.time()
    p = gen.make_workload(3)
    n, g, sc = p.n, p.Hq // p.Hkv, p.eff_scale
    prob = M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, "f32", p.scale, slash_tile=1)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, V = U.device_inputs(p)
    Og = torch.empty((p.B, p.Hq, n, p.dh), dtype=torch.float32, device="cuda")
    t = buf["tiles"]
    M.run_layer(prob, heads, Q, K, V, Og, buf=buf)
    torch.cuda.synchronize()
    assert int(t["status"].item()) == 0
    h = next(h for h, c in enumerate(p.heads) if c.kind == gen.VSLASH)
    vi = buf["vert_idx"][0, h].cpu().numpy()
    si = buf["slash_idx"][0, h].cpu().numpy()
    cols, offs = vi[vi >= 0].astype(np.int64), si[si >= 0].astype(np.int64)
    assert int(t["kept_edges"][0, h].item()) == O.vs_edges(n, cols, offs, 1)
    U.log(f"  exact pairs: head {h} kept edges match ({time.time() - t0:.0f}s)")
    cover = O.slash_offset_set(offs, n, 1)
    rows = np.unique(np.concatenate([p.rows, p.edge_rows])).astype(np.int64)
    q = _f32(p.Q[0, h], p.dtype)
    k = _f32(p.K[0, h // g], p.dtype)
    v = _f32(p.V[0, h // g], p.dtype)
    og = Og[0, h][torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = _row_refs(q, _Widened(k), _Widened(v), rows, lambda i: O.vs_row_keys(i, cols, cover, 1), sc,
                    f"head {h} exact pairs")
    U.compare_output(og, ref, p.dtype, f"128K head {h} exact pairs, {len(rows)} rows")


@pytest.mark.timeout(400)
def test_full_size_single_launch_vs_index():
    """minf_vs_index_fused at the 128K mixed layer, in the launch the bench
    times: the selections of VS heads from two KV groups against the oracle's
    proxy scores, and every VS head's scores against the two-launch path."""
    import torch
    t0 = time.time()
    p = gen.make_workload(3)
    U.log(f"workload {p.name}: generated in {time.time() - t0:.0f}s")
    g = p.Hq // p.Hkv
    prob = M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, "f32", p.scale)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    Q, K, _ = U.device_inputs(p)
    scores = []
    for fn in (M.minf_vs_index_fused, M.minf_vs_index):
        c = torch.zeros((p.B, p.Hq, p.n), dtype=torch.float32, device="cuda")
        r = torch.zeros_like(c)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        if fn is M.minf_vs_index_fused:
            fn(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"], status=st)
        else:
            fn(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"])
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        if not scores:
            vi, si = buf["vert_idx"].cpu().numpy(), buf["slash_idx"].cpu().numpy()
        scores.append((c.cpu().numpy(), r.cpu().numpy()))
    del Q, K
    vs_heads = [h for h, c in enumerate(p.heads) if c.kind == gen.VSLASH]
    assert vs_heads
    for h in vs_heads:
        for x, y, what in ((scores[0][0], scores[1][0], "columns"), (scores[0][1], scores[1][1], "offsets")):
            s = max(float(np.abs(y[0, h]).max()), 1e-30)
            assert np.abs(x[0, h] - y[0, h]).max() <= 1e-5 * s, (h, what)
    checked = [vs_heads[0]] + [h for h in vs_heads if h // g != vs_heads[0] // g][:1]
    for h in checked:
        cfg = p.heads[h]
        q = _f32(p.Q[0, h], p.dtype).astype(np.float64)
        k = _f32(p.K[0, h // g], p.dtype).astype(np.float64)
        c, r = O.vs_proxy_scores(q, k, cfg.last_q, p.eff_scale)
        d1, _ = U.check_selection(vi[0, h][vi[0, h] >= 0], c, cfg.n_vertical, f"head {h} columns")
        d2, _ = U.check_selection(si[0, h][si[0, h] >= 0], r, cfg.n_slash, f"head {h} offsets")
        U.log(f"  head {h}: single-launch selection matches ({d1 + d2} near-tie differences, {time.time() - t0:.0f}s)")
