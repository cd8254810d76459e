"""Choosing which layers keep an indexer (F) and which reuse the nearest
earlier F layer's index set (S), from measured index-set overlaps.

The pages choose the F/S split of an existing model greedily, layer by
layer, on a small calibration batch, scoring each choice by the model's loss
(IndexCache article after VentureBeat (linkstar.cloud), section on the two
deployment routes; IndexCache news article (app.myzaker.com), section
"IndexCache": search which layers to keep by the loss change).  Without a
model or data, the proxy here is how much of each layer's own top-k set the
reused set still contains:

    coverage(pattern) = mean over layers l of  |I_l ∩ I_src(l)| / |I_l|,

src(l) being the nearest F layer at or before l (an F layer covers itself).
The overlaps come from the library's idx_overlap kernel on all-F index sets;
the greedy walk below is host logic.

    python -m long_context_sparse_idx_amd.search [--workload search32k] [--n-f 3]
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Sequence

import numpy as np


def sources(pattern: Sequence[int]) -> list:
    """src(l): the nearest F layer at or before l (pattern[0] must be F)."""
    if not pattern or not pattern[0]:
        raise ValueError("a pattern starts with an F layer")
    out, cur = [], 0
    for l, f in enumerate(pattern):
        if f:
            cur = l
        out.append(cur)
    return out


def coverage(M: np.ndarray, pattern: Sequence[int]) -> float:
    """Mean over layers of M[l, src(l)], M[l, m] = |I_l ∩ I_m| / |I_l|."""
    src = sources(pattern)
    return float(np.mean([M[l, s] for l, s in enumerate(src)]))


def greedy_pattern(M: np.ndarray, n_f: int) -> tuple:
    """Start with every layer F; repeatedly turn into S the F layer (never
    layer 0) whose removal keeps the coverage highest (ties: the lowest
    layer), until n_f F layers remain."""
    L = M.shape[0]
    if not 1 <= n_f <= L:
        raise ValueError("1 <= n_f <= number of layers")
    pat = [1] * L
    while sum(pat) > n_f:
        best, best_l = -1.0, -1
        for l in range(1, L):
            if pat[l]:
                trial = list(pat)
                trial[l] = 0
                c = coverage(M, trial)
                if c > best:
                    best, best_l = c, l
        pat[best_l] = 0
    return tuple(pat)


def best_pattern(M: np.ndarray, n_f: int) -> tuple:
    """The coverage-maximising pattern with n_f F layers, exactly: coverage
    is a sum of per-segment terms (the layers from one F layer up to the
    next read that F layer's set), so a dynamic programme over (segment
    start, F layers left) finds the optimum (ties: the earliest next F).
    The pages' loss is not additive over layers, which is why their search
    is greedy; this overlap proxy admits the exact answer as a reference."""
    L = M.shape[0]
    if not 1 <= n_f <= L:
        raise ValueError("1 <= n_f <= number of layers")
    pre = [np.concatenate([[0.0], np.cumsum(M[:, s])]) for s in range(L)]  # pre[s][e] = sum_{l<e} M[l, s]
    seg = lambda s, e: pre[s][e] - pre[s][s]
    NEG = -1.0
    best = np.full((L + 1, n_f + 1), NEG)
    nxt = np.full((L + 1, n_f + 1), -1, np.int64)
    for s in range(L - 1, -1, -1):
        best[s, 1] = seg(s, L)
        for c in range(2, n_f + 1):
            for e in range(s + 1, L):
                if best[e, c - 1] < 0:
                    continue
                v = seg(s, e) + best[e, c - 1]
                if v > best[s, c] + 1e-12:
                    best[s, c], nxt[s, c] = v, e
    pat = [0] * L
    s, c = 0, n_f
    while s >= 0 and c >= 1:
        pat[s] = 1
        s, c = (int(nxt[s, c]), c - 1) if c > 1 else (-1, 0)
    return tuple(pat)


def overlap_matrix(sets) -> np.ndarray:
    """M[l, m] = sum over rows of |I_l ∩ I_m| / sum over rows of |I_l| for
    index sets [B, T, k] int32 on the GPU (one per layer, all-F)."""
    import torch
    from . import lcsi
    L = len(sets)
    valid = [float((s >= 0).sum().item()) for s in sets]
    M = np.eye(L)
    for l in range(L):
        for m in range(l + 1, L):
            c = float(lcsi.idx_overlap(sets[l], sets[m]).sum(dtype=torch.int64).item())
            M[l, m] = c / max(valid[l], 1.0)
            M[m, l] = c / max(valid[m], 1.0)
    return M


def all_f_index_sets(wl, device="cuda"):
    """Every layer's own top-k sets [B, n_q, k] (the all-F pattern), chunk
    by chunk as the workload prescribes."""
    import torch
    from . import inputs, lcsi
    sets = []
    ws = None
    for l in range(wl.n_layers):
        x = inputs.indexer_inputs(wl, l, device)
        idx = torch.empty((wl.B, wl.n_q, wl.top_k), dtype=torch.int32, device=device)
        for (q0, tq, T_kv) in wl.chunks():
            r0 = q0 - wl.q_pos0
            qs = x["q_scale"][:, r0:r0 + tq] if x["q_scale"] is not None else None
            d = lcsi.indexer_desc(x["q"][:, r0:r0 + tq], x["k"], x["w"][:, r0:r0 + tq], wl.top_k, q0,
                                  k_scale=x["k_scale"], T_kv=T_kv, q_scale=qs)
            need = lcsi.idx_score_topk_ws_bytes(d)
            if ws is None or ws.numel() * 4 < need:
                ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=device)
            lcsi.idx_score_topk(d, idx[:, r0:r0 + tq], ws)
        sets.append(idx)
        del x
    torch.cuda.synchronize()
    return sets


def main(argv=None):
    from . import inputs
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="search32k", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--n-f", type=int, default=None, help="F layers to keep (default: the workload's)")
    args = ap.parse_args(argv)
    wl = inputs.WORKLOADS[args.workload]
    L = wl.n_layers
    n_f = args.n_f or wl.n_f
    M = overlap_matrix(all_f_index_sets(wl))
    fixed = wl.pattern
    greedy = greedy_pattern(M, n_f)
    best = best_pattern(M, n_f)
    name = lambda p: "".join("F" if f else "S" for f in p)
    out = {"workload": wl.name, "layers": L, "n_f": n_f,
           "greedy_pattern": name(greedy), "greedy_coverage": round(coverage(M, greedy), 4),
           "best_pattern": name(best), "best_coverage": round(coverage(M, best), 4),
           "fixed_pattern": name(fixed), "fixed_coverage": round(coverage(M, fixed), 4),
           "adjacent_overlap": [round(float(M[l + 1, l]), 4) for l in range(L - 1)]}
    print(json.dumps(out), flush=True)
    return out


if __name__ == "__main__":
    main()
