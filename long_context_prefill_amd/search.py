"""Offline kernel-aware pattern search on calibration input.

PaperTrace 2.1.2 "MInference", sections 3.1 and 6.3, and blog-zz7
"LLM模型之MInference", section 2.3.1 (Eq. 2): per head, each candidate
pattern (A-shape, Vertical-Slash, Block-Sparse) at each budget approximates
the dense attention of a calibration input; the search keeps, per head, the
configuration that runs fastest on this library's kernels among those whose
output error is acceptable.  The search is offline: it is not on the
per-request path, so it may be slow.

How it runs here:
* every candidate configuration is applied to all heads of the layer at once
  and the four C-ABI calls (index estimation, tile build, attention) run on
  the calibration input; the layer time is measured with HIP events (median
  of ``reps`` runs after one warm-up run), so the time includes the index
  stages the candidate needs;
* each head is compared with dense attention (every head A-shape with no
  sink and a window of n keys, i.e. all j <= i) in two measures, both named
  by section 3.1 of the MInference page:
  - the missed attention mass 1 - m, where m is the mean over rows (and
    batch) of the fraction of the dense softmax that the kept keys carry,
    m_i = exp(lse_i - lse_dense,i) (minf_captured_mass); Eq. 2's L1
    distance between the renormalised and the dense attention row is
    2 (1 - m_i), so this is half the row-mean of Eq. 2's first objective;
  - the relative output error ||O_h - O_dense,h||_F / ||O_dense,h||_F over
    all rows (minf_output_error);
* head h takes, among the candidates whose error in the chosen measure
  (missed mass by default) is at most eps, the one with the least layer
  time; ties go to the earlier candidate of the grid (the grid lists simpler
  configurations first), and the dense candidate, whose errors are 0,
  always qualifies;
* heads are independent, so running the chosen table reproduces, head by
  head, the candidate outputs the errors were measured on; the search runs
  the chosen table once more to measure its time and confirm its errors.

eps is the caller's.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import (MINF_ASHAPE, MINF_BSPARSE, MINF_FORCE_DIAG_BLOCK, MINF_FORCE_FIRST_BLOCK, MINF_VSLASH,
               alloc_buffers, make_heads, minf_bs_index, minf_build_tiles, minf_captured_mass, minf_output_error,
               minf_sparse_attn, minf_vs_index)

Cfg = Tuple[int, int, int, int, int, int, int, int]   # minf_head_cfg field order


def ashape(sink: int, window: int) -> Cfg:
    return (MINF_ASHAPE, sink, window, 0, 0, 0, 0, 0)


def vslash(last_q: int, n_vertical: int, n_slash: int) -> Cfg:
    return (MINF_VSLASH, 0, 0, last_q, n_vertical, n_slash, 0, 0)


def bsparse(topk: int, force: int = MINF_FORCE_FIRST_BLOCK | MINF_FORCE_DIAG_BLOCK) -> Cfg:
    return (MINF_BSPARSE, 0, 0, 0, 0, 0, topk, force)


def dense(n: int) -> Cfg:
    return ashape(0, n)


def describe(c: Cfg) -> str:
    if c[0] == MINF_ASHAPE:
        return f"ashape(sink={c[1]},window={c[2]})"
    if c[0] == MINF_VSLASH:
        return f"vslash(last_q={c[3]},v={c[4]},s={c[5]})"
    return f"bsparse(k={c[6]},force={c[7]})"


def default_grid(n: int) -> List[Cfg]:
    """Budgets of each pattern, simpler (cheaper) first; the dense candidate
    last.  Budgets that do not fit n are dropped."""
    nq = (n + 63) // 64
    grid: List[Cfg] = []
    for sink, window in ((64, 256), (128, 1024), (128, 4096)):
        if window < n:
            grid.append(ashape(sink, window))
    for v, s in ((250, 500), (500, 2000), (1000, 4096)):
        if v <= n and s <= n:
            grid.append(vslash(64, v, s))
    for k in (8, 16, 32, 64):
        if k < nq:
            grid.append(bsparse(k))
    grid.append(dense(n))
    return grid


def choose(rel_err: Sequence[Sequence[float]], times_ms: Sequence[float], eps: float) -> List[int]:
    """Per head: the candidate of least time among those with error <= eps
    (ties to the earlier candidate); -1 if none qualifies."""
    out = []
    for errs in rel_err:
        best = -1
        for c, e in enumerate(errs):
            if e <= eps and (best < 0 or times_ms[c] < times_ms[best]):
                best = c
        out.append(best)
    return out


class _Runner:
    """Runs one layer (all four calls) for a head table on fixed inputs."""

    def __init__(self, prob, Q, K, V, O, lse, stream=None):
        self.prob, self.Q, self.K, self.V, self.O, self.lse = prob, Q, K, V, O, lse
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.err = torch.empty(2 * prob.B * prob.Hq, dtype=torch.float64, device=Q.device)
        self.mass = torch.empty(prob.B * prob.Hq, dtype=torch.float64, device=Q.device)

    def run(self, table: Sequence[Cfg], reps: int) -> float:
        heads = make_heads(table)
        buf = alloc_buffers(self.prob, heads)
        t = buf["tiles"]

        def step():
            minf_vs_index(self.prob, heads, self.Q, self.K, buf["vert_idx"], buf["slash_idx"], None, None,
                          buf["ws"], stream=self.stream)
            minf_bs_index(self.prob, heads, self.Q, self.K, buf["blk_idx"], buf["blk_cnt"], buf["ws"],
                          stream=self.stream)
            minf_build_tiles(self.prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"], t,
                             buf["ws"], stream=self.stream)
            minf_sparse_attn(self.prob, heads, self.Q, self.K, self.V, buf["blk_idx"], buf["blk_cnt"], t, self.O,
                             self.lse, buf["ws"], stream=self.stream)

        step()
        ms = []
        for _ in range(max(1, reps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            step()
            e1.record(self.stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        if int(t["status"].item()) != 0:
            raise RuntimeError(f"device status {int(t['status'].item())} for table {[describe(c) for c in table]}")
        ms.sort()
        return ms[len(ms) // 2]

    def rel_errors(self, O_ref) -> List[float]:
        """Per head h: ||O_h - O_ref,h|| / ||O_ref,h||, summed over the batch."""
        minf_output_error(self.prob, self.O, O_ref, self.err, stream=self.stream)
        e = self.err.cpu().tolist()
        B, Hq = self.prob.B, self.prob.Hq
        out = []
        for h in range(Hq):
            d2 = sum(e[2 * (b * Hq + h)] for b in range(B))
            r2 = sum(e[2 * (b * Hq + h) + 1] for b in range(B))
            out.append(math.sqrt(d2 / r2) if r2 > 0 else (0.0 if d2 == 0 else math.inf))
        return out

    def missed_mass(self, lse_ref) -> List[float]:
        """Per head h: 1 - mean over rows and batch of exp(lse - lse_ref)."""
        minf_captured_mass(self.prob, self.lse, lse_ref, self.mass, stream=self.stream)
        m = self.mass.cpu().tolist()
        B, Hq, n = self.prob.B, self.prob.Hq, self.prob.n
        return [1.0 - sum(m[b * Hq + h] for b in range(B)) / (B * n) for h in range(Hq)]


def search(prob, Q, K, V, grid: Optional[Sequence[Cfg]] = None, eps: float = 0.05, reps: int = 3,
           measure: str = "mass", stream=None) -> Dict:
    """Run the search on one calibration layer (device tensors Q [B,Hq,n,dh],
    K/V [B,Hkv,n,dh] in the problem's input type).  measure: "mass" (missed
    attention mass) or "output" (relative output error) decides the choice.
    Returns the candidates, their layer times, both per-head error tables
    [head][candidate], the choice per head, and the chosen table with its own
    time and errors."""
    if measure not in ("mass", "output"):
        raise ValueError(f"measure must be 'mass' or 'output', not {measure!r}")
    n, Hq = prob.n, prob.Hq
    grid = list(grid) if grid is not None else default_grid(n)
    if dense(n) not in grid:
        grid.append(dense(n))
    odt = torch.float32 if prob.out_dtype == 0 else torch.bfloat16
    O = torch.empty((prob.B, Hq, n, prob.dh), dtype=odt, device=Q.device)
    lse = torch.empty((prob.B, Hq, n), dtype=torch.float32, device=Q.device)
    run = _Runner(prob, Q, K, V, O, lse, stream)
    dense_ms = run.run([dense(n)] * Hq, reps)
    O_dense, lse_dense = O.clone(), lse.clone()
    times, rel, miss = [], [], []
    for c in grid:
        # (the dense candidate runs again too: its errors against the first
        # dense run are 0, as the kernels are deterministic)
        times.append(run.run([c] * Hq, reps))
        rel.append(run.rel_errors(O_dense))
        miss.append(run.missed_mass(lse_dense))
    rel_h = [[rel[c][h] for c in range(len(grid))] for h in range(Hq)]
    miss_h = [[miss[c][h] for c in range(len(grid))] for h in range(Hq)]
    choice = choose(miss_h if measure == "mass" else rel_h, times, eps)
    table = [grid[c] for c in choice]
    table_ms = run.run(table, reps)
    return {
        "eps": eps,
        "measure": measure,
        "candidates": [describe(c) for c in grid],
        "cfgs": [list(c) for c in grid],
        "times_ms": times,
        "dense_ms": dense_ms,
        "missed_mass": miss_h,
        "rel_err": rel_h,
        "choice": choice,
        "table": [describe(c) for c in table],
        "table_cfgs": [list(c) for c in table],
        "table_ms": table_ms,
        "table_missed_mass": run.missed_mass(lse_dense),
        "table_rel_err": run.rel_errors(O_dense),
    }
