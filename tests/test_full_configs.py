"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (runner.Workload: one run_layer_group call per chunk).

The oracle recomputes sampled rows one by one: rows at p in {0, 1, k-2,
k-1, k, k+1, last} and spread positions (chunk boundaries included).  Each
sampled row checks the GPU scores (1e-2 relative, floor 1e-3 of the row
max), the index set (identical except near-ties within that tolerance of
the k-th value) and every layer's attention output on the GPU's index set
(max-abs <= 2e-2).  Large K/V arrays reach the oracle as the gathered rows
the index set names (indices renumbered, order kept), which leaves its
arithmetic unchanged."""
import numpy as np
import pytest
import torch

import oracle
from helpers import ATTN_ATOL, ATTN_ROW_REL, attn_row_rel, bf16_to_f64, check_index_sets, check_scores, log
from long_context_sparse_idx_amd import inputs, lcsi
from long_context_sparse_idx_amd.runner import Workload

pytestmark = pytest.mark.gpu


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sample_positions(wl, extra=12):
    lo, hi = wl.q_pos0, wl.q_pos0 + wl.n_q - 1
    k = wl.top_k
    cand = {lo, lo + 1, k - 2, k - 1, k, k + 1, hi}
    for (q0, tq, _) in wl.chunks():
        cand |= {q0, q0 + tq - 1}
    cand |= set(np.linspace(lo, hi, extra).astype(int).tolist())
    pos = sorted(p for p in cand if lo <= p <= hi)
    if len(pos) > 24:  # keep the chunk-boundary and special rows, thin the rest
        keep = {lo, lo + 1, k - 2, k - 1, k, k + 1, hi}
        rest = [p for p in pos if p not in keep]
        pos = sorted(keep & set(pos) | set(rest[:: max(1, len(rest) // 16)]))
    return pos


def gpu_scores(run: Workload, layer, b, pos):
    """Scores of sampled rows: re-run the F layer's indexer on each row alone
    (SCORES_ONLY); a row's scores do not depend on its chunk."""
    wl = run.wl
    x = run.idx_in[layer]
    out = []
    for p in pos:
        r = p - wl.q_pos0
        d = lcsi.indexer_desc(x["q"][b:b + 1, r:r + 1], x["k"][b:b + 1], x["w"][b:b + 1, r:r + 1], wl.top_k, p,
                              k_scale=x["k_scale"][b:b + 1] if x["k_scale"] is not None else None, T_kv=p + 1,
                              q_scale=x["q_scale"][b:b + 1, r:r + 1] if x["q_scale"] is not None else None)
        ws = torch.empty(lcsi.idx_score_topk_ws_bytes(d) // 4, dtype=torch.float32, device="cuda")
        lcsi.idx_score_topk(d, None, ws, flags=lcsi.LCSI_SCORES_ONLY)
        torch.cuda.synchronize()
        out.append(ws[:p + 1].cpu().numpy())
    return out


def gathered_attn_oracle(run: Workload, layer, b, pos, g_idx):
    """Oracle attention of sampled rows on the GPU's index sets, with K/V cut
    down to the rows those sets name."""
    wl = run.wl
    x = run.attn_in[layer]
    rows = torch.tensor([p - wl.q_pos0 for p in pos], device="cuda")
    q = u16(x["q"][b].index_select(0, rows))
    valid = g_idx[g_idx >= 0]
    uniq = np.unique(valid)
    remap = np.full(g_idx.shape, -1, np.int32)
    lut = {int(v): i for i, v in enumerate(uniq)}
    for i in range(g_idx.shape[0]):
        for j in range(g_idx.shape[1]):
            if g_idx[i, j] >= 0:
                remap[i, j] = lut[int(g_idx[i, j])]
    sel = torch.from_numpy(uniq.astype(np.int64)).cuda()
    K = u16(x["k"][b].index_select(0, sel))
    if wl.kv_shared:
        V = (K, wl.D_v)
    else:
        V = u16(x["v"][b].index_select(0, sel))
    return oracle.attn(q, K, V, remap, run.tau)


def check_workload(name, n_slots=None, batches=(0,), allf_overlap=False):
    wl = inputs.WORKLOADS[name]
    nf = wl.n_f
    slots = nf if n_slots is None else n_slots
    log(f"[full] {name}: B={wl.B} n_q={wl.n_q} T_kv={wl.T_kv} pattern={wl.pattern} slots={slots}")
    run = Workload(wl, n_slots=slots, log=log)
    plan = run.plan()
    run.step(plan)
    torch.cuda.synchronize()
    pos = sample_positions(wl)
    rows_t = torch.tensor([p - wl.q_pos0 for p in pos], device="cuda")
    swaps = 0
    worst_rel = 0.0
    for b in batches:
        for fi, layer in enumerate(run.pattern_f):
            x = run.idx_in[layer]
            g_idx = run.cache[fi % slots, b].index_select(0, rows_t).cpu().numpy()
            keys = x["k"][b].cpu().numpy() if wl.key_fp8 else u16(x["k"][b])
            ks = x["k_scale"][b].cpu().numpy() if wl.key_fp8 else None
            if wl.q_fp8:
                q = x["q"][b].index_select(0, rows_t).cpu().numpy()
                qs = x["q_scale"][b].index_select(0, rows_t).cpu().numpy()
            else:
                q, qs = u16(x["q"][b].index_select(0, rows_t)), None
            w = x["w"][b].index_select(0, rows_t).cpu().numpy()
            rS, r_idx = oracle.score_select(q, w, keys, np.array(pos, np.int64), wl.top_k, k_scale=ks, q_scale=qs)
            gS = gpu_scores(run, layer, b, pos)
            for i, p in enumerate(pos):
                check_scores(gS[i], rS[i, :p + 1], f"{name} b={b} F-layer {layer} p={p}")
                swaps += check_index_sets(g_idx[i], r_idx[i], rS[i, :p + 1], wl.top_k,
                                          f"{name} b={b} F-layer {layer} p={p}")
            # every layer that reads this slot: its own attention on these indices
            users = [l for l in range(wl.n_layers)
                     if l >= layer and (fi + 1 == nf or l < run.pattern_f[fi + 1])]
            for l in users:
                o = gathered_attn_oracle(run, l, b, pos, g_idx)
                g = u16(run.outs[l][b].index_select(0, rows_t))
                err = float(np.abs(bf16_to_f64(g) - bf16_to_f64(o)).max())
                rel = float(attn_row_rel(g, o).max())
                worst_rel = max(worst_rel, rel)
                assert err <= ATTN_ATOL, f"{name} b={b} layer {l}: max abs err {err}"
                assert rel <= ATTN_ROW_REL, f"{name} b={b} layer {l}: row-relative err {rel}"
        log(f"  b={b}: {len(pos)} rows x {nf} F layers checked, near-tie swaps {swaps}, "
            f"attention row-relative err max {worst_rel:.3e} (bound {ATTN_ROW_REL})")
    return run


def test_full_prefill32k():
    run = check_workload("prefill32k")
    # adjacent-layer overlap of the generator's per-layer queries (statistic)
    wl = run.wl
    allf = tuple(1 for _ in range(wl.n_layers))
    run2 = Workload(wl, f_layers=range(wl.n_layers), n_slots=wl.n_layers)
    run2.step(run2.plan(allf))
    torch.cuda.synchronize()
    a = run2.cache[0, 0, ::257].cpu().numpy()
    ov = []
    for l in range(1, wl.n_layers):
        c = run2.cache[l, 0, ::257].cpu().numpy()
        ov.append(float(np.mean([np.intersect1d(a[i][a[i] >= 0], c[i][c[i] >= 0]).size / max(1, (a[i] >= 0).sum())
                                 for i in range(a.shape[0])])))
    log(f"  prefill32k overlap |I_l & I_0| / k for l=1..3: {[round(v, 3) for v in ov]}")


def test_full_prefill200k():
    check_workload("prefill200k")


def test_full_decode131k():
    check_workload("decode131k", batches=(0, 13, 31))


def test_full_prefill1m():
    check_workload("prefill1m")


def test_full_decode1m():
    check_workload("decode1m", batches=(0, 7))


def test_full_prefill1m_fp8_queries():
    check_workload("prefill1m_q8")


def test_full_decode1m_fp8_queries():
    check_workload("decode1m_q8", batches=(0, 5))


def test_full_prefill200k_fp8():
    check_workload("prefill200k_q8")
