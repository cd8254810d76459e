"""The fused candidate pass of the indexer (scores at or above a sampled
threshold kept per row, selection on those) against the unfused path and
the oracle.

The fused pass must give the same indices as writing every score row and
selecting from it: the candidates are the same fp32 scores, and every score
that reaches a row's k-th largest is a candidate whenever the row's count is
at least k.  Rows whose sample misjudges them (fewer than k candidates, or
more than the 16384 slots) are rescored in full; both cases are forced here
from the inputs (equal keys: every score ties, so every row overflows; keys
made large exactly on the sampled tiles: the threshold lands above the
row's k-th score).  Long rows with few sampled scores per row (16 heads)
cover candidate counts above what the LDS lists hold.

Unsettled rows are listed by the fused pass; the first 64 are rescored by
the split-key kernel (many workgroups per row), and only when the list
overflows do whole workgroups rescore their rows.  Both are covered.

The counts are read back from the workspace (right after the score rows) to
check that each case took the path it is meant to."""
import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_idx_amd import lcsi
from helpers import bits, log

pytestmark = pytest.mark.gpu

CAP = 16384          # candidate slots per row
RMAX = 64            # unsettled rows a rescoring launch takes from the list


def run_both(d, B, T_q, k):
    """(fused idx, unfused idx, fused counts) as host arrays."""
    n_ws = lcsi.idx_score_topk_ws_bytes(d)
    assert n_ws > lcsi.idx_score_topk_ws_bytes(d, lcsi.LCSI_UNFUSED), "fused pass not planned"
    ws = torch.empty(n_ws // 4, dtype=torch.float32, device="cuda")
    idx = torch.empty((B, T_q, k), dtype=torch.int32, device="cuda")
    idx_u = torch.empty_like(idx)
    lcsi.idx_score_topk(d, idx, ws)
    torch.cuda.synchronize()
    rows_bytes = (B * T_q * lcsi.score_ld(d.T_kv) * 4 + 255) // 256 * 256
    cnt = ws.view(torch.int32)[rows_bytes // 4:rows_bytes // 4 + B * T_q].cpu().numpy().reshape(B, T_q)
    lcsi.idx_score_topk(d, idx_u, ws, flags=lcsi.LCSI_UNFUSED)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), idx_u.cpu().numpy(), cnt


def int_inputs(B, T_q, T_kv, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-8, 9, (B, T_q, H, D), generator=g).to(torch.float32)
    k = torch.randint(-8, 9, (B, T_kv, D), generator=g).to(torch.float32)
    w = (2.0 ** torch.randint(-3, 1, (B, T_q, H), generator=g)).to(torch.float32)
    return q, k, w


def encode(fmt, q, k, B, T_q, T_kv, H, seed):
    g = torch.Generator().manual_seed(seed + 1)
    ks = qs = None
    if fmt == "bf16":
        kd = k.to(torch.bfloat16)
    else:
        kd = k.to(torch.float8_e4m3fn).view(torch.uint8)
        ks = (2.0 ** torch.randint(-2, 2, (B, T_kv), generator=g)).to(torch.float32)
    if fmt == "qk8":
        qd = q.to(torch.float8_e4m3fn).view(torch.uint8)
        qs = (2.0 ** torch.randint(-2, 2, (B, T_q, H), generator=g)).to(torch.float32)
    else:
        qd = q.to(torch.bfloat16)
    return qd, kd, ks, qs


# (H, D, fmt, T_q, q_pos0): rows from below to well above 16384 keys, the
# workgroup count at or above 256 so the prefill kernel (and the fused
# pass) runs, ragged last workgroup
CASES = [
    (64, 128, "bf16", 2043, 15000),
    (64, 128, "k8", 2043, 15000),
    (64, 128, "qk8", 2043, 15000),
    (32, 128, "bf16", 4100, 14000),
    (16, 64, "bf16", 8200, 12000),
    (64, 64, "k8", 2050, 30000),
]


@pytest.mark.parametrize("H,D,fmt,T_q,q_pos0", CASES)
def test_fused_matches_unfused_and_oracle(H, D, fmt, T_q, q_pos0):
    B, k = 1, 2048
    T_kv = q_pos0 + T_q
    seed = 7 * H + D + len(fmt)
    log(f"fused H={H} D={D} {fmt} T_q={T_q} q_pos0={q_pos0}")
    q, kk, w = int_inputs(B, T_q, T_kv, H, D, seed)
    qd, kd, ks, qs = encode(fmt, q, kk, B, T_q, T_kv, H, seed)
    # (device copies held in locals: the descriptor keeps raw pointers)
    dq, dk, dw = qd.cuda(), kd.cuda(), w.cuda()
    dks = ks.cuda() if ks is not None else None
    dqs = qs.cuda() if qs is not None else None
    d = lcsi.indexer_desc(dq, dk, dw, k, q_pos0, k_scale=dks, q_scale=dqs)
    idx, idx_u, cnt = run_both(d, B, T_q, k)
    assert np.array_equal(idx, idx_u)
    n = q_pos0 + np.arange(T_q) + 1
    # rows of workgroups whose longest row has at most CAP keys keep every
    # score; sampled rows keep between k and CAP (misjudged rows aside)
    qpb = 8 * 64 // H
    wg_max = np.minimum((np.arange(T_q) // qpb + 1) * qpb, T_q) + q_pos0
    full = wg_max <= CAP
    assert np.array_equal(cnt[0, full], n[full])
    sampled = cnt[0, ~full]
    ok = (sampled >= k) & (sampled <= CAP)
    log(f"  sampled rows {sampled.size}: counts {sampled.min()}..{sampled.max()}, "
        f"median {int(np.median(sampled))}, misjudged {int((~ok).sum())}")
    assert ok.mean() > 0.99
    # integer-exact inputs: the oracle's indices, exactly, on sampled rows
    rows = np.unique(np.linspace(0, T_q - 1, 12).astype(np.int64))
    if fmt == "bf16":
        qh, kh, qsh, ksh = bits(qd[0, rows]), bits(kd[0]), None, None
    else:
        kh, ksh = kd[0].numpy(), ks[0].numpy()
        if fmt == "qk8":
            qh, qsh = qd[0, rows].numpy(), qs[0, rows].numpy()
        else:
            qh, qsh = bits(qd[0, rows]), None
    _, r_idx = oracle.score_select(qh, w[0, rows].numpy(), kh, q_pos0 + rows, k, k_scale=ksh,
                                   want_scores=False, q_scale=qsh)
    assert np.array_equal(idx[0, rows], r_idx)


def test_fused_all_ties_overflow_and_rescore():
    """Every key equal: each row's scores all tie, every sampled row keeps all
    of its keys (more than the slots) and is rescored; the top-k is then the
    first k positions."""
    B, H, D, k = 1, 64, 128, 2048
    T_q, q_pos0 = 2048, 17000
    T_kv = q_pos0 + T_q
    g = torch.Generator().manual_seed(11)
    q = torch.randn((B, T_q, H, D), generator=g).to(torch.bfloat16)
    key = torch.randn((1, 1, D), generator=g)
    kk = key.expand(B, T_kv, D).contiguous().to(torch.bfloat16)
    w = torch.rand((B, T_q, H), generator=g) + 0.1
    dq, dk, dw = q.cuda(), kk.cuda(), w.cuda()
    d = lcsi.indexer_desc(dq, dk, dw, k, q_pos0)
    idx, idx_u, cnt = run_both(d, B, T_q, k)
    assert np.array_equal(idx, idx_u)
    assert (cnt > CAP).all(), "every row should overflow its slots"
    assert (idx == np.arange(k, dtype=np.int32)[None, None, :]).all()


@pytest.mark.parametrize("n_hot", [4, 64])
def test_fused_threshold_too_high_rescore(n_hot):
    """Keys scaled up exactly on the tiles the fused pass samples, in the
    first n_hot batch entries: the sampled threshold lands above each of
    their rows' k-th score, the rows keep fewer than k candidates and are
    rescored -- 32 rows: from the list of unsettled rows, by the split-key
    kernel; 512 rows: more than the list holds, by whole workgroups.  One
    workgroup per batch entry (8 rows), 256 entries: of the n_tiles whole
    128-key tiles below the first row's position, a workgroup samples ns
    spread evenly (tile i * n_tiles // ns), ns = ceil(24 n / (k 128))
    clamped to 4..32 (about 24 sampled scores above the k-th)."""
    B, H, D, k = 256, 64, 128, 2048
    T_q, q_pos0 = 8, 20000
    T_kv = q_pos0 + T_q
    g = torch.Generator().manual_seed(12)
    qd = torch.randint(-8, 9, (B, T_q, H, D), generator=g, dtype=torch.int8).to(torch.bfloat16)
    kd = torch.randint(-8, 9, (B, T_kv, D), generator=g, dtype=torch.int8).to(torch.bfloat16)
    n_tiles = (q_pos0 + 1) // 128
    ns = min(32, max(4, -(-24 * (q_pos0 + 1) // (k * 128))))
    for i in range(ns):
        t = i * n_tiles // ns
        kd[:n_hot, t * 128:(t + 1) * 128] *= 16  # integers up to 128: exact in bf16
    w = torch.ones((B, T_q, H))
    dq, dk, dw = qd.cuda(), kd.cuda(), w.cuda()
    d = lcsi.indexer_desc(dq, dk, dw, k, q_pos0)
    idx, idx_u, cnt = run_both(d, B, T_q, k)
    assert np.array_equal(idx, idx_u)
    low = cnt < k
    log(f"  rows with fewer than k candidates: {int(low.sum())} of {low.size}")
    assert low[:n_hot].all() and not low[n_hot:].any()
    assert (n_hot * T_q <= RMAX) == (n_hot == 4)
    for b in (0, n_hot - 1, n_hot):
        rows = np.array([0, 5])
        _, r_idx = oracle.score_select(bits(qd[b, rows]), w[b, rows].numpy(), bits(kd[b]), q_pos0 + rows, k,
                                       want_scores=False)
        assert np.array_equal(idx[b, rows], r_idx), b


def test_fused_long_rows_stream_candidates():
    """16 heads: at most 1024 sampled scores per row; rows of ~600K keys
    then keep about 8K candidates, often more than the LDS lists hold
    (8192), so the selection streams them from memory (a few rows overflow
    their slots and are rescored from the list)."""
    B, H, D, k = 256, 16, 64, 2048
    T_q, q_pos0 = 32, 600000
    T_kv = q_pos0 + T_q
    g = torch.Generator().manual_seed(13)
    q = torch.randn((B, T_q, H, D), generator=g).to(torch.bfloat16)
    kk = torch.randn((1, T_kv, D), generator=g).to(torch.bfloat16)
    w = torch.rand((B, T_q, H), generator=g) + 0.1
    dq, dk, dw = q.cuda(), kk.cuda().expand(B, T_kv, D), w.cuda()
    d = lcsi.indexer_desc(dq, dk, dw, k, q_pos0)
    assert d.k_sb == 0
    idx, idx_u, cnt = run_both(d, B, T_q, k)
    assert np.array_equal(idx, idx_u)
    streamed = (cnt > 8192) & (cnt <= CAP)
    log(f"  counts {cnt.min()}..{cnt.max()}, streamed rows {int(streamed.sum())}, "
        f"overflow {int((cnt > CAP).sum())}, below k {int((cnt < k).sum())}")
    assert streamed.sum() > 100


@pytest.mark.parametrize("k", [1, 64, 700])
def test_fused_small_top_k(k):
    """Sampled rows with a small top-k (the sampled rank r falls to a few
    samples): the candidates still settle the rows and match the unfused
    path; integer-exact rows match the oracle."""
    B, H, D = 1, 64, 128
    T_q, q_pos0 = 2048, 20000
    T_kv = q_pos0 + T_q
    q, kk, w = int_inputs(B, T_q, T_kv, H, D, 100 + k)
    qd, kd = q.to(torch.bfloat16), kk.to(torch.bfloat16)
    dq, dk, dw = qd.cuda(), kd.cuda(), w.cuda()
    d = lcsi.indexer_desc(dq, dk, dw, k, q_pos0)
    idx, idx_u, cnt = run_both(d, B, T_q, k)
    assert np.array_equal(idx, idx_u)
    ok = (cnt >= k) & (cnt <= CAP)
    log(f"  k={k}: counts {cnt.min()}..{cnt.max()}, unsettled {int((~ok).sum())}")
    assert ok.mean() > 0.99
    rows = np.array([0, 1000, 2047])
    _, r_idx = oracle.score_select(bits(qd[0, rows]), w[0, rows].numpy(), bits(kd[0]), q_pos0 + rows, k,
                                   want_scores=False)
    assert np.array_equal(idx[0, rows], r_idx)
