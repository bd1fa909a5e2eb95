"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (whole layer: Vertical-Slash index,
Block-Sparse index, tile build, sparse attention, fp32 output).

For every workload, one head of each pattern kind present is checked:
* its index against the oracle's: Vertical-Slash columns and offsets, and
  every query block's Block-Sparse selection, identical except candidates
  whose oracle score lies within 1e-4 relative of the k-th threshold;
* its kept edges, exactly, from the GPU's own index sets;
* its output rows against the oracle's restricted softmax over the GPU's own
  index sets (max-abs 1e-2, mean-abs 1e-3 for bf16 inputs): all rows up to
  32K tokens; above that the 4096 seeded sampled rows plus the edge rows
  for the first checked head and 512 of them for the others.
"""
import math
import time

import numpy as np
import pytest

from tests.conftest import gpu_available
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import long_context_prefill_amd as M  # noqa: E402
from oracle import minf_oracle as O  # noqa: E402
from synth import gen  # noqa: E402


def _checked_heads(p):
    seen, out = set(), []
    for h, c in enumerate(p.heads):
        if c.kind not in seen:
            seen.add(c.kind)
            out.append(h)
    if len(out) == 1:
        out.append(p.Hq - 1)          # a second head from another KV group
    return out


def _f32(x, dtype):
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _row_refs(q, k, v, rows, keys_fn, scale, what):
    """Oracle rows (float64 arithmetic on exactly widened inputs), on threads."""
    from concurrent.futures import ThreadPoolExecutor

    def one(i):
        keys = keys_fn(int(i))
        return O.attend_row_keys(q[i].astype(np.float64), k, v, keys, scale)

    out = np.zeros((len(rows), v.shape[1]))
    t0 = time.time()
    with ThreadPoolExecutor(12) as ex:
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


@pytest.mark.timeout(400)
@pytest.mark.parametrize("w", [2, 3, 4, 5])
def test_full_size_layer(w):
    import torch
    t0 = time.time()
    p = gen.make_workload(w)
    U.log(f"workload {p.name}: generated in {time.time() - t0:.0f}s")
    n, nq = p.n, (p.n + 63) // 64
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
        rows_all = np.arange(n, dtype=np.int64)
    else:
        rows_all = np.unique(np.concatenate([p.rows, p.edge_rows])).astype(np.int64)
    vi = buf["vert_idx"].cpu().numpy()
    si = buf["slash_idx"].cpu().numpy()
    ke = t["kept_edges"].cpu().numpy()
    del Q, K, V

    for num, h in enumerate(_checked_heads(p)):
        cfg = p.heads[h]
        b = 0
        kv = h // g
        what = f"{p.name} head {h} ({gen.KIND_NAMES[cfg.kind]})"
        q = _f32(p.Q[b, h], p.dtype)
        k = _f32(p.K[b, kv], p.dtype)
        v = _f32(p.V[b, kv], p.dtype)
        # ---- index against the oracle's
        if cfg.kind == gen.VSLASH:
            c, r = O.vs_proxy_scores(q.astype(np.float64), k.astype(np.float64), cfg.last_q, sc)
            cols, offs = vi[b, h][vi[b, h] >= 0], si[b, h][si[b, h] >= 0]
            d1, e1 = U.check_selection(cols, c, cfg.n_vertical, f"{what} columns")
            d2, e2 = U.check_selection(offs, r, cfg.n_slash, f"{what} offsets")
            U.log(f"  {what}: index matches ({d1 + d2} near-tie differences)")
            cover = O.slash_offset_set(offs, n, 64)
            assert int(ke[b, h]) == O.vs_edges(n, cols, offs, 64)
            xs = np.nonzero(cover)[0] - 63
            colset = np.asarray(cols, dtype=np.int64)

            def keys_fn(i, xs=xs, colset=colset):
                j = 64 * (i // 64) - xs
                j = j[(j >= 0) & (j <= i)]
                return np.union1d(j, colset[colset <= i])
            mask_fn = lambda rr, nk: O.vs_mask(rr, nk, n, cols, offs, 64, cover)
        elif cfg.kind == gen.BSPARSE:
            bi = buf["blk_idx"][b, h].cpu().numpy()
            bc = buf["blk_cnt"][b, h].cpu().numpy()
            J = [bi[u, :bc[u]].astype(np.int64) for u in range(nq)]
            scores = O.bs_block_scores(q.astype(np.float64), k.astype(np.float64), sc)
            nd = 0
            for u in range(nq):
                row = scores[u, :u + 1].copy()
                if cfg.force_flags & gen.FORCE_FIRST_BLOCK:
                    row[0] = np.inf
                if cfg.force_flags & gen.FORCE_DIAG_BLOCK:
                    row[u] = np.inf
                d, _ = U.check_selection(J[u], row, cfg.topk_blocks, f"{what} block {u}")
                nd += d
            U.log(f"  {what}: index matches ({nd} near-tie differences)")
            del scores
            assert int(ke[b, h]) == O.bs_edges(n, J)
            keys_fn = lambda i, J=J: O.bs_row_keys(i, J)
            mask_fn = lambda rr, nk: O.bs_mask(rr, nk, J)
        else:
            assert int(ke[b, h]) == int(O.ashape_row_counts(n, cfg.sink, cfg.window).sum())
            keys_fn = lambda i, cfg=cfg: O.ashape_row_keys(i, cfg.sink, cfg.window)
            mask_fn = lambda rr, nk, cfg=cfg: O.ashape_mask(rr, nk, cfg.sink, cfg.window)
        # ---- output rows against the oracle's restricted softmax
        rows = rows_all if (num == 0 or p.rows is None) else rows_all[:: max(1, len(rows_all) // 512)]
        og = Og[b, h][torch.from_numpy(rows).cuda()].cpu().numpy()
        if p.rows is None:
            ref, _ = O.attend_rows(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), rows,
                                   mask_fn, sc)
        else:
            ref = _row_refs(q, _Widened(k), _Widened(v), rows, keys_fn, sc, what)
        U.compare_output(og, ref, p.dtype, f"{what}, {len(rows)} rows")
        U.log(f"  {what}: done ({time.time() - t0:.0f}s)")


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
        fn(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], c, r, buf["ws"])
        torch.cuda.synchronize()
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
