"""Benchmark: one MInference-style sparse prefill layer on one MI355X.

A step is one pass of the whole hot path on resident inputs: Vertical-Slash
index, Block-Sparse index, tile build and sparse attention (all HIP kernels
of libminf, called through the C interface).  The workload is the 128K mixed
layer: B=1, Hq=32, Hkv=8, n=131072, dh=128, bf16, seeded synthetic inputs
with planted sinks and periodic slashes; 16 Vertical-Slash heads
(last_q=64, 1000 verticals, 6096 slashes), 8 Block-Sparse heads (top-100)
and 8 A-shape heads (sink 128, window 4096).

Prints one JSON line.  The metric is milliseconds per layer (index +
attention, lower is better); the line also carries the per-stage split, the
kept-edge TFLOP/s of the attention kernel against the bf16 matrix peak
(roofline), and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill ms/layer @128K (index+attn) and kept-edge TFLOP/s vs bf16 peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E

# HBM traffic of one attention-kernel launch on the 128K mixed layer, from
# two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch), each scaled by what the same counter reads for a plain
# device copy of known size (bench.py --copy-mib).  Valid only for the kernel
# sources they were taken from: the hash covers them, and a mismatch (or
# None) reports null.
ATTN_KERNEL = "attn_bf16_d128_kernel"
ATTN_SOURCES = ["long_context_prefill_amd/csrc/attn_bf16.hip", "long_context_prefill_amd/csrc/common.h",
                "long_context_prefill_amd/csrc/kernels.h", "include/minf.h"]
ATTN_TRAFFIC = {"workload": "n128k_h32kv8_d128_bf16_mixed", "sources": "84f88fa25b3e4d54",
                "fetch_kib": 24463163.52, "fetch_factor": 1048576 / 524302.1,
                "write_kib": 2112678.95, "write_factor": 1048576 / 1048576.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def index_bytes(p):
    """Algorithmic HBM bytes of the index stage: K read once per KV group
    that has a VS head, the sampled Q rows, c and r written and read; Q of
    the BS heads and K of their groups read once, J written."""
    from synth import gen
    g = p.Hq // p.Hkv
    el = 2 if p.dtype == "bf16" else 4
    row = p.dh * el
    vs = [h for h, c in enumerate(p.heads) if c.kind == gen.VSLASH]
    bs = [h for h, c in enumerate(p.heads) if c.kind == gen.BSPARSE]
    nq = (p.n + 63) // 64
    b = 0
    b += len({h // g for h in vs}) * p.n * row
    b += sum(min(p.heads[h].last_q, p.n) * row + 4 * p.n * 4 for h in vs)
    b += len(bs) * p.n * row + len({h // g for h in bs}) * p.n * row
    b += sum(nq * min(p.heads[h].topk_blocks, nq) * 4 for h in bs)
    return b * p.B


def sources_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_traffic(workload):
    t = ATTN_TRAFFIC
    if t is None or t["workload"] != workload or t["sources"] != sources_hash(ATTN_SOURCES):
        return None
    return t["fetch_kib"] * 1024 * t["fetch_factor"] + t["write_kib"] * 1024 * t["write_factor"]


def computed_pairs(p, t, buf):
    """(query row, key) pairs the attention kernel computes: 64 x 32 per
    chunk of every query block (sink and window chunks, slash-span chunks,
    packed chunks of span tails, gathered-column chunks, two chunks per
    selected block).  kept / computed
    is the tile efficiency E_h / E~_h."""
    import numpy as np
    from synth import gen
    nq = (p.n + 63) // 64
    u = np.arange(nq, dtype=np.int64)
    total = 0
    cc = t["chunk_cnt"].cpu().numpy() if "chunk_cnt" in t else None
    pk = t["pk_cnt"].cpu().numpy() if "pk_cnt" in t else None
    colc = t["col_cnt"].cpu().numpy() if "col_cnt" in t else None
    bc = buf["blk_cnt"].cpu().numpy()
    for b in range(p.B):
        for h, c in enumerate(p.heads):
            if c.kind == gen.VSLASH:
                chunks = (cc[b, h].astype(np.int64) + pk[b, h].astype(np.int64) +
                          (colc[b, h].astype(np.int64) + 31) // 32)
            elif c.kind == gen.BSPARSE:
                chunks = 2 * bc[b, h].astype(np.int64)
            else:
                g, w = min(c.sink, p.n), min(c.window, p.n)
                sink_len = np.minimum(g, np.minimum(64 * u + 64, p.n))
                wlo = np.maximum(np.maximum(g, 64 * u - w + 1), 0)
                whi = np.minimum(64 * u + 63, p.n - 1)
                chunks = (sink_len + 31) // 32 + np.where((w > 0) & (whi >= wlo), (whi - wlo + 32) // 32, 0)
            total += int(chunks.sum())
    return total * 64 * 32


def copy_probe(mib, reps):
    """A plain device copy of known size, for scaling the memory counters."""
    import torch
    x = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": mib << 20, "reps": reps}), flush=True)


def measured_peaks():
    """The box's own ceilings, measured beside the vendor figures: a bf16
    matrix product (torch.mm, 8192^3, hipBLASLt) and a device-to-device copy
    of 2 GiB (read + write bytes), medians of 10 event-timed runs each."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)

    def med(fn, reps=10):
        for _ in range(3):
            fn()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return sorted(ms)[reps // 2]
    t_mm = med(lambda: torch.mm(a, b))
    t_cp = med(lambda: y.copy_(x))
    out = {"bf16_gemm_tflops": round(2.0 * n ** 3 / (t_mm * 1e-3) / 1e12, 1),
           "copy_gbs": round(2.0 * x.numel() * 4 / (t_cp * 1e-3) / 1e9, 1),
           "what": "torch.mm bf16 8192x8192x8192 and a 2 GiB device copy (bytes read + written), "
                   "median of 10 event-timed runs each"}
    del a, b, x, y
    torch.cuda.empty_cache()
    return out


def cpu_baseline(p, workers):
    """The oracle as it stands, timed on a bounded sample of the same layer:
    full index estimation of half of the heads (kinds in the layer's
    proportions) and the restricted softmax on R sampled rows of those heads;
    extrapolated (labelled) to the whole layer."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import minf_oracle as O
    from synth import gen
    kinds = {}
    for h, c in enumerate(p.heads):
        kinds.setdefault(c.kind, []).append(h)
    sample = []
    for k, hs in kinds.items():
        sample += hs[:max(1, len(hs) // 2)]
    R = min(4096, p.n)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(p.n, R, replace=False))
    sc = p.eff_scale
    g = p.Hq // p.Hkv

    def one(h):
        q = O.widen(p.Q[0, h], p.dtype)
        k = O.widen(p.K[0, h // g], p.dtype)
        v = O.widen(p.V[0, h // g], p.dtype)
        t0 = time.perf_counter()
        res = O.head_index(q, k, p.heads[h], p.n, sc)
        t1 = time.perf_counter()
        O.attend_rows(q, k, v, rows, res.mask_fn, sc)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    nw = min(workers, len(sample))
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), ThreadPoolExecutor(nw) as ex:
        times = list(ex.map(one, sample))
    wall = time.perf_counter() - t0
    # per-head CPU seconds, extrapolated per kind to every head and every row
    est = 0.0
    for h, (ti, ta) in zip(sample, times):
        same = len(kinds[p.heads[h].kind]) / sum(1 for s in sample if p.heads[s].kind == p.heads[h].kind)
        est += same * (ti + ta * p.n / R)
    ms_layer = 1000.0 * est / nw          # the same thread count working on the whole layer
    return {"value": round(ms_layer, 1), "unit": "ms/layer (extrapolated)", "cores": nw, "kind": "oracle",
            "sample": f"{len(sample)} of {p.Hq} heads (kinds in layer proportion): full index + {R} sampled "
                      f"query rows of restricted softmax; wall {wall:.1f}s on {nw} threads; extrapolated to "
                      f"all heads and all {p.n} rows"}


def dense_heads(Hq, n):
    """The dense causal baseline on the same kernels: every head A-shape with
    no sink and a window of n keys, i.e. all j <= i."""
    from synth import gen
    return [gen.ashape(0, n)] * Hq


def time_layer(M, prob, heads, Q, K, V, O_, steps, warmup, index=True, flush=None):
    """Median event-timed ms of (index stages,) tile build and attention."""
    import numpy as np
    import torch
    buf = M.alloc_buffers(prob, heads)
    t = buf["tiles"]
    stream = torch.cuda.current_stream()

    def step():
        if index:
            M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"])
            M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
        M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"], t,
                           buf["ws"])
        M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], t, O_, None, buf["ws"])

    for _ in range(warmup):
        step()
    ms = []
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    if int(t["status"].item()) != 0:
        raise RuntimeError(f"device status {int(t['status'].item())}")
    kept = int(t["kept_edges"].sum().item())
    del buf
    return float(np.median(ms)), kept


def pattern_search(a, n):
    """The offline kernel-aware pattern search on a synthetic calibration layer
    (KV groups with local, planted and clustered structure), B=1, Hq=32,
    Hkv=8, dh=128, bf16, length a.search; one JSON line."""
    import numpy as np
    import torch
    import long_context_prefill_amd as M
    from long_context_prefill_amd import search as S
    from synth import gen
    t0 = time.time()
    p = gen.make_calibration(n=n, Hq=32, Hkv=8, dh=128, dtype="bf16")
    log(f"generated {p.name} in {time.time() - t0:.1f}s")
    conv = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    prob = M.make_problem(1, 32, 8, n, 128, "bf16", "f32")
    t0 = time.time()
    res = S.search(prob, conv(p.Q), conv(p.K), conv(p.V), eps=a.search_eps, reps=max(1, a.steps))
    log(f"search in {time.time() - t0:.1f}s")
    kinds = {}
    for c in res["table_cfgs"]:
        k = ("ashape", "vslash", "bsparse")[c[0]]
        kinds[k] = kinds.get(k, 0) + 1
    by_group = {}
    for h, ch in enumerate(res["choice"]):
        g = p.meta["group_kinds"][h // 4]
        by_group.setdefault(g, []).append(res["candidates"][ch])
    out = {
        "metric": "offline pattern search: layer ms of the chosen per-head table vs dense, error <= eps",
        "config": {"workload": p.name, "B": 1, "n": n, "Hq": 32, "Hkv": 8, "dh": 128,
                   "structure_by_kv_group": p.meta["group_kinds"]},
        "data": "synthetic calibration layer, seeded",
        "eps": res["eps"],
        "candidates": res["candidates"],
        "times_ms": [round(t, 4) for t in res["times_ms"]],
        "dense_ms": round(res["dense_ms"], 4),
        "table_ms": round(res["table_ms"], 4),
        "speedup_vs_dense": round(res["dense_ms"] / res["table_ms"], 3),
        "table_kinds": kinds,
        "choice_by_structure": by_group,
        "measure": res["measure"],
        "max_table_missed_mass": round(max(res["table_missed_mass"]), 5),
        "max_table_rel_err": round(max(res["table_rel_err"]), 5),
        "best_missed_mass_by_structure": {
            g: [round(min(res["missed_mass"][h][c] for h in range(32) if p.meta["group_kinds"][h // 4] == g), 4)
                for c in range(len(res["candidates"]))]
            for g in sorted(set(p.meta["group_kinds"]))},
        "timing": "median of the timed runs after one warm-up run, warm caches; each candidate on all heads",
    }
    return out


RAGGED_LENS = [65536, 8192, 32768, 4096, 16384, 49152, 12288, 24576]


def ragged_batch(a):
    """Eight prompts of 4K-64K tokens (planted inputs, the 128K layer's mixed
    pattern table), packed without padding through minf_prefill_ragged,
    against the same prompts padded to the longest as one B = 8 batch
    through the four calls; one JSON line."""
    import numpy as np
    import torch
    import long_context_prefill_amd as M
    from synth import gen
    Hq, Hkv, dh = 32, 8, 128
    table = gen.pattern_table(3)
    heads = M.make_heads(table)
    lens = RAGGED_LENS
    n_max, T = max(lens), sum(lens)
    t0 = time.time()
    samples = [gen.generate(f"req{i}_n{n}", 1, Hq, Hkv, n, dh, "bf16", table, 5000 + i, dist="planted")
               for i, n in enumerate(lens)]
    log(f"generated {len(lens)} requests ({T} tokens) in {time.time() - t0:.1f}s")
    conv = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    cat = lambda xs: conv(np.concatenate([x[0].reshape(-1) for x in xs]))
    Qp, Kp, Vp = cat([s.Q for s in samples]), cat([s.K for s in samples]), cat([s.V for s in samples])
    prob_r = M.make_problem(len(lens), Hq, Hkv, n_max, dh, "bf16", "f32")
    O_r = torch.empty(Hq * T * dh, dtype=torch.float32, device="cuda")
    kept_r = torch.zeros((len(lens), Hq), dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_r = torch.empty(M.minf_ragged_ws_bytes(prob_r, heads, lens), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        fn()
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    ms_r = timed(lambda: M.minf_prefill_ragged(prob_r, heads, lens, Qp, Kp, Vp, O_r, None, kept_r, status, ws_r),
                 max(1, a.steps))
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    kept = int(kept_r.sum().item())
    del Qp, Kp, Vp, O_r, ws_r
    torch.cuda.empty_cache()
    # the same prompts padded to the longest (zeros after each prompt)
    Qd = torch.zeros((len(lens), Hq, n_max, dh), dtype=torch.int16, device="cuda")
    Kd = torch.zeros((len(lens), Hkv, n_max, dh), dtype=torch.int16, device="cuda")
    Vd = torch.zeros((len(lens), Hkv, n_max, dh), dtype=torch.int16, device="cuda")
    for b, s in enumerate(samples):
        n = s.n
        Qd[b, :, :n] = conv(s.Q[0])
        Kd[b, :, :n] = conv(s.K[0])
        Vd[b, :, :n] = conv(s.V[0])
    del samples
    prob_p = M.make_problem(len(lens), Hq, Hkv, n_max, dh, "bf16", "f32")
    buf = M.alloc_buffers(prob_p, heads)
    O_p = torch.empty((len(lens), Hq, n_max, dh), dtype=torch.float32, device="cuda")
    ms_p = timed(lambda: M.run_layer(prob_p, heads, Qd, Kd, Vd, O_p, buf=buf), max(1, a.steps))
    out = {
        "metric": "ragged batch prefill ms (8 prompts, 4K-64K tokens) vs the same batch padded to the longest",
        "config": {"workload": "ragged8_planted_h32kv8_d128_bf16_mixed", "lens": lens, "tokens": T, "Hq": Hq,
                   "Hkv": Hkv, "dh": dh, "heads": "the 128K layer's table: 16 vertical-slash, 8 block-sparse, "
                                                  "8 A-shape"},
        "data": "synthetic, seeded (planted sinks + periodic slashes), resident in HBM",
        "ragged_ms": round(ms_r, 3),
        "padded_ms": round(ms_p, 3),
        "padded_over_ragged": round(ms_p / ms_r, 3),
        "ragged_tokens_per_s": round(T / (ms_r * 1e-3), 1),
        "ragged_kept_edges": kept,
        "ragged_kept_edge_tflops": round(4 * dh * kept / (ms_r * 1e-3) / 1e12, 1),
        "timing": "median of the timed runs after one warm-up run, warm caches; whole path (index, tiles, attention)",
    }
    return out


def crossover(a):
    """Sparse layer (index + attention, the 128K mixed pattern table) against
    the dense causal baseline over sequence lengths, on planted inputs of
    each length; one JSON line."""
    import numpy as np
    import torch
    import long_context_prefill_amd as M
    from synth import gen
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    rows = []
    for n in [int(x) for x in a.crossover.split(",")]:
        t0 = time.time()
        p = gen.generate(f"crossover_n{n}", 1, 32, 8, n, 128, "bf16", gen.pattern_table(3), 1003,
                         dist="planted", sample_rows=4096)
        log(f"generated n={n} in {time.time() - t0:.1f}s")
        conv = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        Q, K, V = conv(p.Q), conv(p.K), conv(p.V)
        O_ = torch.empty((1, 32, n, 128), dtype=torch.float32, device="cuda")
        prob = M.make_problem(1, 32, 8, n, 128, "bf16", "f32", 0.0)
        ms_s, kept_s = time_layer(M, prob, M.make_heads(p.heads), Q, K, V, O_, a.steps, a.warmup, True, flush)
        ms_d, kept_d = time_layer(M, prob, M.make_heads(dense_heads(32, n)), Q, K, V, O_, a.steps, a.warmup,
                                  False, flush)
        rows.append({"n": n, "sparse_ms": round(ms_s, 3), "dense_ms": round(ms_d, 3),
                     "speedup": round(ms_d / ms_s, 3), "sparse_kept_edges": kept_s, "dense_edges": kept_d,
                     "dense_tflops": round(4 * 128 * kept_d / (ms_d * 1e-3) / 1e12, 1)})
        log(json.dumps(rows[-1]))
        del Q, K, V, O_
    wins = [r["n"] for r in rows if r["speedup"] > 1.0]
    print(json.dumps({"metric": "sparse vs dense causal prefill ms/layer by sequence length",
                      "unit": "ms/layer", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
                      "config": {"workload": "planted B=1 Hq=32 Hkv=8 dh=128, 128K mixed pattern table",
                                 "lengths": [r["n"] for r in rows]},
                      "rows": rows, "sparse_wins_from_n": min(wins) if wins else None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the 1 GiB cache-flushing write before each timed step")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--crossover", default="",
                    help="comma-separated lengths: time the sparse layer against the dense causal baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense causal baseline")
    ap.add_argument("--no-exact", action="store_true", help="skip the exact slash pairs (slash_tile=1) layer")
    ap.add_argument("--no-search", action="store_true", help="skip the pattern search summary (32K calibration layer)")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged batch summary")
    ap.add_argument("--no-vs-single", action="store_true",
                    help="skip timing the Vertical-Slash estimate alone (two-launch vs single-launch proxy)")
    ap.add_argument("--search", type=int, default=0,
                    help="only run the offline pattern search on a calibration layer of this length")
    ap.add_argument("--search-eps", type=float, default=0.05, help="error bound of the pattern search")
    ap.add_argument("--ragged", action="store_true",
                    help="only time a ragged batch of 8 requests against the same batch padded to its longest")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the box's bf16 GEMM and copy ceilings")
    ap.add_argument("--peaks", action="store_true", help="only measure the box's bf16 GEMM and copy ceilings")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (memory-counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(sharding over KV-head groups is a design note, not code).", file=sys.stderr)
        sys.exit(2)

    if a.copy_mib:
        copy_probe(a.copy_mib, max(1, a.steps))
        return
    if a.peaks:
        print(json.dumps(measured_peaks()), flush=True)
        return
    if a.crossover:
        crossover(a)
        return
    if a.search:
        print(json.dumps(pattern_search(a, a.search)), flush=True)
        return
    if a.ragged:
        print(json.dumps(ragged_batch(a)), flush=True)
        return

    import numpy as np
    import torch
    import long_context_prefill_amd as M
    from synth import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    t0 = time.time()
    p = gen.make_workload(a.workload)
    log(f"generated {p.name} in {time.time() - t0:.1f}s")
    conv = (lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()) if p.dtype == "bf16" \
        else (lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda())
    Q, K, V = conv(p.Q), conv(p.K), conv(p.V)
    prob = M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, a.out_dtype, p.scale)
    heads = M.make_heads(p.heads)
    buf = M.alloc_buffers(prob, heads)
    odt = torch.float32 if a.out_dtype == "f32" else torch.bfloat16
    O_ = torch.empty((p.B, p.Hq, p.n, p.dh), dtype=odt, device="cuda")
    t = buf["tiles"]
    stream = torch.cuda.current_stream()

    stages = ["vs_index", "bs_index", "build_tiles", "sparse_attn"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        M.minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"])
        mark(1)
        M.minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"])
        mark(2)
        M.minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"], t,
                           buf["ws"])
        mark(3)
        M.minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], t, O_, None, buf["ws"])
        mark(4)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    if int(t["status"].item()) != 0:
        raise RuntimeError(f"device status {int(t['status'].item())}")

    # Timed steps.  Before each one a 1 GiB write evicts L2 and the MALL
    # (outside the events), so the layer starts with cold caches, as it would
    # after the projections of a real layer.  The events bracket each call;
    # the library's own event pair brackets the attention kernel alone.
    flush = None if a.no_flush else torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def timed(k, do_flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(k)]
        M.minf_timing_start(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(k):
            if do_flush:
                flush.fill_(float(s_))
            step(evs[s_])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = M.minf_timing_read(k)
        per = [[evs[s_][i].elapsed_time(evs[s_][i + 1]) for i in range(4)] for s_ in range(k)]
        return wall, per, kern

    wall, per, kern = timed(a.steps, flush is not None)
    if int(t["status"].item()) != 0:
        raise RuntimeError(f"device status {int(t['status'].item())}")
    warm = timed(a.steps, False)[1] if flush is not None else None
    ms_wall = 1000.0 * wall / a.steps
    layer = np.array([sum(x) for x in per])
    st = {k: float(np.median([x[i] for x in per])) for i, k in enumerate(stages)}
    ms_step = float(np.median(layer))
    ms_index = float(np.median([x[0] + x[1] + x[2] for x in per]))
    ms_attn = st["sparse_attn"]
    ms_kernel = float(np.mean(kern))

    kept = int(t["kept_edges"].sum().item())
    flops = 4.0 * p.dh * kept * p.B if p.B == 1 else 4.0 * p.dh * kept
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    kern_tflops = flops / (ms_kernel * 1e-3) / 1e12
    ib = index_bytes(p)
    idx_gbs = ib / (ms_index * 1e-3) / 1e9
    per_kind = {}
    ke = t["kept_edges"].cpu().numpy()
    for h, c in enumerate(p.heads):
        per_kind.setdefault(gen.KIND_NAMES[c.kind], 0)
        per_kind[gen.KIND_NAMES[c.kind]] += int(ke[:, h].sum())
    dense = p.B * p.Hq * p.n * (p.n + 1) // 2
    computed = computed_pairs(p, t, buf)

    dense_bl = None
    if not a.no_dense:
        t0 = time.time()
        ms_d, kept_d = time_layer(M, prob, M.make_heads(dense_heads(p.Hq, p.n)), Q, K, V, O_, 3, 1, False, flush)
        dense_bl = {"ms": round(ms_d, 3), "kept_edges": kept_d,
                 "tflops": round(4 * p.dh * kept_d / (ms_d * 1e-3) / 1e12, 1),
                 "speedup_of_sparse": round(ms_d / ms_step, 3),
                 "what": "same inputs, every head A-shape(sink 0, window n) = all j <= i; tile build + attention, "
                         "median of 3 cache-flushed steps"}
        log(f"dense baseline in {time.time() - t0:.1f}s")

    exact = None
    if not a.no_exact and "vslash" in per_kind:
        t0 = time.time()
        prob1 = M.make_problem(p.B, p.Hq, p.Hkv, p.n, p.dh, p.dtype, a.out_dtype, p.scale, slash_tile=1)
        ms_e, kept_e = time_layer(M, prob1, heads, Q, K, V, O_, 3, 1, True, flush)
        exact = {"ms": round(ms_e, 3), "kept_edges": kept_e,
                 "what": "same layer with slash_tile=1 (Eq. 5 pairs: row i keeps key j iff i-j is a selected "
                         "offset or j a selected column); index + tiles + attention, median of 3 cache-flushed "
                         "steps"}
        log(f"exact slash pairs in {time.time() - t0:.1f}s")

    vs_fused = None
    if "vslash" in per_kind and not a.no_vs_single:
        # the Vertical-Slash estimate alone, warm: the two-launch path the layer
        # uses against the single-launch proxy (minf_vs_index_fused)
        vs_status = torch.zeros(1, dtype=torch.int32, device="cuda")

        def vs_ms(fn, reps=20):
            kw = {"status": vs_status} if fn is M.minf_vs_index_fused else {}
            fn(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"], stream=stream, **kw)
            ms = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], None, None, buf["ws"], stream=stream, **kw)
                e1.record(stream)
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            return sorted(ms)[reps // 2]
        two, one = vs_ms(M.minf_vs_index), vs_ms(M.minf_vs_index_fused)
        torch.cuda.synchronize()
        if int(vs_status.item()) != 0:
            raise RuntimeError("minf_vs_index_fused: a bounded wait ran out (MINF_DEV_WAIT_EXHAUSTED)")
        vs_fused = {"two_launch_ms": round(two, 4), "single_launch_ms": round(one, 4),
                    "what": "Vertical-Slash estimate (proxy, fold, column and slash sums, top-k) alone, warm, "
                            "median of 20: minf_vs_index (the layer's path) vs minf_vs_index_fused"}
    search = None
    if not a.no_search:
        t0 = time.time()
        r = pattern_search(argparse.Namespace(steps=3, search_eps=a.search_eps), 32768)
        search = {k: r[k] for k in ("config", "eps", "measure", "dense_ms", "table_ms", "speedup_vs_dense",
                                    "table_kinds", "max_table_missed_mass", "max_table_rel_err")}
        search["what"] = ("offline kernel-aware pattern search on a 32K calibration layer (local, planted and "
                          "clustered KV groups); bench.py --search 32768 prints every candidate")
        log(f"pattern search in {time.time() - t0:.1f}s")
    ragged = None
    if not a.no_ragged:
        t0 = time.time()
        r = ragged_batch(argparse.Namespace(steps=3))
        ragged = {k: r[k] for k in ("config", "ragged_ms", "padded_ms", "padded_over_ragged", "ragged_tokens_per_s",
                                    "ragged_kept_edge_tflops")}
        log(f"ragged batch in {time.time() - t0:.1f}s")

    peaks = None
    if not a.no_peaks:
        t0 = time.time()
        peaks = measured_peaks()
        peaks["attn_frac_of_measured_gemm"] = round(kern_tflops / peaks["bf16_gemm_tflops"], 4)
        peaks["index_frac_of_measured_copy"] = round(idx_gbs / peaks["copy_gbs"], 4)
        log(f"measured peaks in {time.time() - t0:.1f}s")

    cpu = None
    if not a.no_cpu_baseline:
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        t0 = time.time()
        cpu = cpu_baseline(p, min(16, cores))
        log(f"cpu baseline in {time.time() - t0:.1f}s")

    out = {
        "metric": METRIC,
        "value": round(ms_step, 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_wall, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic, seeded (planted sinks + periodic slashes), resident in HBM",
        "config": {"workload": p.name, "B": p.B, "n": p.n, "Hq": p.Hq, "Hkv": p.Hkv, "dh": p.dh,
                   "heads": "16 vertical-slash (64/1000/6096), 8 block-sparse (top-100), 8 A-shape (128/4096)"
                   if a.workload == 3 else str(sorted(per_kind)),
                   "out_dtype": a.out_dtype},
        "timing": ("median over the timed steps of the event-timed layer (index + attention); "
                   + ("each step starts after a 1 GiB cache-flushing write, which ms_per_step (wall clock) "
                      "includes" if flush is not None else "warm caches")),
        "ms_layer_min_max": [round(float(layer.min()), 3), round(float(layer.max()), 3)],
        "ms_layer_warm": round(float(np.median([sum(x) for x in warm])), 3) if warm else None,
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "ms_index": round(ms_index, 4),
        "ms_attn": round(ms_attn, 4),
        "kept_edges": kept,
        "kept_edges_by_kind": per_kind,
        "dense_causal_edges": dense,
        "computed_pairs": computed,
        "tile_efficiency": round(kept / computed, 4) if computed else None,
        "kept_edge_tflops": round(attn_tflops, 2),
        "frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "index_gbs": round(idx_gbs, 1),
        "index_frac_hbm": round(idx_gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": attn_traffic(p.name), "traffic_unit": "HBM bytes per launch",
                     "kernel": ATTN_KERNEL if (p.dtype == "bf16" and p.dh == 128) else "attn_kernel",
                     "per_launch_flops": flops, "avg_launch_ms": round(ms_kernel, 4),
                     "launches_timed": len(kern)},
        "measured_peaks": peaks,
        "dense_baseline": dense_bl,
        "exact_slash_pairs": exact,
        "vs_single_launch": vs_fused,
        "pattern_search": search,
        "ragged_batch": ragged,
        "cpu_baseline": cpu,
        "context": "pages: up to 10x prefill speedup over dense on an A100 (another machine and workload)",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
