"""Loop-only restatement of the oracle for tiny inputs (n up to ~130).

TEST INFRASTRUCTURE ONLY (same rule as minf_oracle.py).  Pure Python loops,
no vectorisation, written directly from the set definitions so that the
vectorised oracle can be checked against an independent code path:

* A-shape, Eq. 3 of PaperTrace 2.1.2 "MInference" (section 2);
* Vertical-Slash, Eq. 5 (section 2.1) with each slash expanded to the
  t x t tile of the query block (t = 1 gives Eq. 5 itself);
* Block-Sparse, Eq. 6 with mean-pooled block scores (section 2);
* the proxy of section 6.2 and the restricted softmax of Eq. 2.
"""
from __future__ import annotations

import math

ASHAPE, VSLASH, BSPARSE = 0, 1, 2
FORCE_FIRST_BLOCK, FORCE_DIAG_BLOCK = 1, 2


def dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def topk(scores, k):
    """First k of the candidates ordered by (score desc, index asc), sorted."""
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    return sorted(order[:min(k, len(scores))])


def ashape_set(i, sink, window):
    a = set(range(0, min(sink - 1, i) + 1))
    b = set(range(max(0, i - window + 1), i + 1))
    return a | b


def vs_set(i, cols, offs, t):
    u = i // t
    out = set()
    for c in cols:
        if c <= i:
            out.add(c)
    for d in offs:
        for j in range(t * u - d, t * u + t - d):
            if 0 <= j <= i:
                out.add(j)
    return out


def bs_set(i, J, block=64):
    out = set()
    for j in range(i + 1):
        if j // block in J[i // block]:
            out.add(j)
    return out


def vs_scores(q, k, last_q, scale):
    n = len(q)
    L = min(last_q, n)
    c = [0.0] * n
    r = [0.0] * n
    for i in range(n - L, n):
        s = [scale * dot(q[i], k[j]) for j in range(i + 1)]
        m = max(s)
        z = sum(math.exp(x - m) for x in s)
        for j in range(i + 1):
            a = math.exp(s[j] - m) / z
            c[j] += a
            r[i - j] += a
    return c, r


def block_mean(x, u, block):
    rows = x[u * block:min(len(x), (u + 1) * block)]
    dh = len(x[0])
    return [sum(row[d] for row in rows) / len(rows) for d in range(dh)]


def bs_index(q, k, topk_blocks, force, scale, block=64):
    n = len(q)
    nb = (n + block - 1) // block
    qb = [block_mean(q, u, block) for u in range(nb)]
    kb = [block_mean(k, v, block) for v in range(nb)]
    J = []
    for u in range(nb):
        row = [scale * dot(qb[u], kb[v]) for v in range(u + 1)]
        if force & FORCE_FIRST_BLOCK:
            row[0] = math.inf
        if force & FORCE_DIAG_BLOCK:
            row[u] = math.inf
        J.append(set(topk(row, topk_blocks)))
    return J


def attend(q, k, v, i, keys, scale):
    """(o_i, LSE_i) of Eq. 2 restricted to `keys`."""
    dh = len(v[0])
    if not keys:
        return [0.0] * dh, -math.inf
    s = {j: scale * dot(q[i], k[j]) for j in keys}
    m = max(s.values())
    w = {j: math.exp(s[j] - m) for j in keys}
    z = sum(w.values())
    o = [sum(w[j] * v[j][d] for j in keys) / z for d in range(dh)]
    return o, m + math.log(z)


def head(q, k, v, cfg, scale, slash_tile=64, block=64):
    """Index, per-row sets, outputs and kept edges of one head.

    cfg = (kind, sink, window, last_q, n_vertical, n_slash, topk_blocks, force).
    """
    kind, sink, window, last_q, nv, ns, kb, ff = cfg
    n = len(q)
    info = {}
    if kind == ASHAPE:
        sets = [ashape_set(i, sink, window) for i in range(n)]
    elif kind == VSLASH:
        c, r = vs_scores(q, k, last_q, scale)
        cols, offs = topk(c, nv), topk(r, ns)
        info.update(cols=cols, offs=offs, c=c, r=r)
        sets = [vs_set(i, cols, offs, slash_tile) for i in range(n)]
    else:
        J = bs_index(q, k, kb, ff, scale, block)
        info.update(J=[sorted(x) for x in J])
        sets = [bs_set(i, J, block) for i in range(n)]
    outs = [attend(q, k, v, i, sets[i], scale) for i in range(n)]
    info.update(sets=sets, o=[o for o, _ in outs], lse=[l for _, l in outs],
                edges=sum(len(s) for s in sets))
    return info
