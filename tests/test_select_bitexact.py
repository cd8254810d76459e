"""GPU top-k on given fp32 score rows (LCSI_SCORES_PRESET) must be
byte-identical to the oracle's selection: same positions, ascending, same
-1 padding.  Rows cover every path of the kernel: n <= k, whole row in LDS,
the sampled-threshold pass, and the exact streaming fallback (heavy ties,
all-equal rows, +-0, monotone rows); for few long rows also lists longer
than usual (recent positions scoring higher) and more candidates than the
final select holds in registers (a tied plateau)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_idx_amd import lcsi
from helpers import log

pytestmark = pytest.mark.gpu


def run_select(S_rows: np.ndarray, B: int, T_q: int, T_kv: int, q_pos0: int, k: int):
    """S_rows: float32 [B*T_q, n_max]; returns GPU idx [B*T_q, k]."""
    ld = lcsi.score_ld(T_kv)
    d = lcsi.preset_desc(B, T_q, T_kv, q_pos0, k)
    # the score rows first; few long rows also use the space after them
    ws = torch.zeros(max(B * T_q * ld, lcsi.idx_score_topk_ws_bytes(d, lcsi.LCSI_SCORES_PRESET) // 4), dtype=torch.float32, device="cuda")
    wsv = ws[:B * T_q * ld].view(B * T_q, ld)
    wsv[:, :S_rows.shape[1]] = torch.from_numpy(S_rows).cuda()
    idx = torch.full((B, T_q, k), -7, dtype=torch.int32, device="cuda")
    lcsi.idx_score_topk(d, idx, ws, flags=lcsi.LCSI_SCORES_PRESET)
    torch.cuda.synchronize()
    return idx.view(B * T_q, k).cpu().numpy()


def compare(S_rows, B, T_q, T_kv, q_pos0, k, name):
    log(f"[select] case={name} B={B} T_q={T_q} T_kv={T_kv} q_pos0={q_pos0} k={k}")
    g = run_select(S_rows, B, T_q, T_kv, q_pos0, k)
    n = np.array([q_pos0 + t + 1 for _ in range(B) for t in range(T_q)], np.int64)
    r = oracle.select(S_rows, n, k)
    bad = np.nonzero((g != r).any(axis=1))[0]
    assert bad.size == 0, f"{name}: rows {bad[:5]} differ; first: gpu {g[bad[0]][:8]} oracle {r[bad[0]][:8]}"


def rows(rng, B, T_q, T_kv, kind):
    n = T_kv
    R = B * T_q
    if kind == "normal":
        return rng.standard_normal((R, n)).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 5, (R, n)).astype(np.float32)
    if kind == "equal":
        return np.full((R, n), 0.75, np.float32)
    if kind == "signed_zero":
        x = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], np.float32), (R, n))
        return x.astype(np.float32)
    if kind == "increasing":
        return np.tile(np.arange(n, dtype=np.float32), (R, 1))
    if kind == "decreasing":
        return np.tile(-np.arange(n, dtype=np.float32), (R, 1))
    if kind == "positive":  # indexer-like: positive, concentrated
        return (2.0 + 0.4 * rng.standard_normal((R, n))).astype(np.float32)
    if kind == "recent":  # the last 6144 positions score higher: a few long candidate lists
        x = rng.standard_normal((R, n)).astype(np.float32)
        x[:, -6144:] += 1.0
        return x
    if kind == "plateau":  # 5 % of the entries tie at the top: more candidates than a select holds in registers
        x = rng.standard_normal((R, n)).astype(np.float32)
        x[rng.random((R, n)) < 0.05] = 10.0
        return x
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "positive", "ties", "equal", "signed_zero", "increasing",
                                  "decreasing", "recent", "plateau"])
@pytest.mark.parametrize("shape", [
    (2, 6, 40000, 39994, 2048),   # sampled-threshold path (and fallback for ties)
    (1, 6, 16384, 16378, 2048),   # whole row in LDS
    (1, 70, 70, 0, 64),           # n <= k, then LDS path (tiny workload's k)
    (1, 3, 100000, 99997, 1000),  # k not a power of two
    (3, 2, 20000, 19998, 1),      # k = 1
    (4, 1, 300001, 300000, 2048), # few long rows: segment filters + final select
    (1, 2, 70000, 69998, 2048),   # few long rows, 64 segments
])
def test_select_bitexact(kind, shape):
    B, T_q, T_kv, q_pos0, k = shape
    # (a seed that does not depend on the interpreter's string hashing, so a
    # failing case can be rerun from its log line)
    rng = np.random.default_rng(zlib.crc32(repr((kind,) + shape).encode()))
    S = rows(rng, B, T_q, T_kv, kind)
    compare(S, B, T_q, T_kv, q_pos0, k, kind)


def test_select_on_oracle_score_matrix():
    """The oracle's own fp32 score matrix of a real indexer workload."""
    from long_context_sparse_idx_amd import inputs
    import dataclasses
    wl = dataclasses.replace(inputs.WORKLOADS["prefill32k"], n_q=8, q_pos0=20000 - 8, T_kv=20000)
    x = inputs.indexer_inputs(wl, 0, "cpu")
    from helpers import bits
    q = bits(x["q"][0])
    pos = np.arange(wl.q_pos0, wl.q_pos0 + wl.n_q)
    S, r_idx = oracle.score_select(q, x["w"][0].numpy(), bits(x["k"][0]), pos, wl.top_k)
    compare(S, 1, wl.n_q, wl.T_kv, wl.q_pos0, wl.top_k, "oracle-scores")
