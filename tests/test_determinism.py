"""Determinism of the library's results.

* Decode: the same sequences decoded at B = 1, 8, 32 and 64 give
  byte-identical index sets (split-key scoring, few-row selection) and
  byte-identical attention outputs, although the calls differ in how they
  share out the work (key ranges and segments per workgroup, heads per
  workgroup: 16, 32 or 64).  A second identical call gives the same bytes.
* Prefill: one chunk run twice gives identical bytes; the same rows as one
  chunk or as two smaller chunks give identical index sets and outputs.
Outputs are also checked against the oracle on a few rows, so identical bytes
cannot come from a call that wrote nothing."""
import numpy as np
import pytest
import torch

import oracle
from helpers import ATTN_ATOL, bf16_to_f64, bits, check_index_sets, log
from long_context_sparse_idx_amd import lcsi

pytestmark = pytest.mark.gpu

H_I, D_I, H_Q, DQK, DV, TOPK = 64, 128, 64, 576, 512, 2048


def make_decode(n_seq, n_kv, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    dev = "cuda"
    q = torch.randn(n_seq, 1, H_I, D_I, generator=g, device=dev).div_(8).to(torch.bfloat16)
    k = torch.randn(n_seq, n_kv, D_I, generator=g, device=dev).div_(8).to(torch.bfloat16)
    w = torch.rand(n_seq, 1, H_I, generator=g, device=dev)
    qa = torch.randn(n_seq, 1, H_Q, DQK, generator=g, device=dev).to(torch.bfloat16)
    kv = torch.randn(n_seq, n_kv, DQK, generator=g, device=dev).to(torch.bfloat16)
    return q, k, w, qa, kv


def decode_call(x, lo, hi, n_kv):
    """Indexer + attention for sequences lo..hi-1 as one call."""
    q, k, w, qa, kv = (t[lo:hi] for t in x)
    B = hi - lo
    d = lcsi.indexer_desc(q, k, w, TOPK, n_kv - 1)
    ws = torch.empty(lcsi.idx_score_topk_ws_bytes(d) // 4 + 1, dtype=torch.float32, device="cuda")
    idx = torch.full((B, 1, TOPK), -9, dtype=torch.int32, device="cuda")
    lcsi.idx_score_topk(d, idx, ws)
    out = torch.full((B, 1, H_Q, DV), float("nan"), dtype=torch.bfloat16, device="cuda")
    a = lcsi.attn_desc(qa, kv, kv[..., :DV], out, TOPK, n_kv - 1, DQK ** -0.5)
    lcsi.sparse_attn(a, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), bits(out)


def test_decode_is_batch_independent():
    n_seq, n_kv = 64, 40000
    log(f"[determinism] decode: {n_seq} sequences of {n_kv} keys, B in 64/32/8/1")
    x = make_decode(n_seq, n_kv, seed=11)
    ref_idx, ref_out = decode_call(x, 0, n_seq, n_kv)
    again_idx, again_out = decode_call(x, 0, n_seq, n_kv)
    assert np.array_equal(ref_idx, again_idx) and np.array_equal(ref_out, again_out), "B=64 run to run"
    for B in (32, 8):
        for lo in range(0, n_seq, B):
            gi, go = decode_call(x, lo, lo + B, n_kv)
            assert np.array_equal(gi, ref_idx[lo:lo + B]), f"indices differ at B={B}, sequences {lo}.."
            assert np.array_equal(go, ref_out[lo:lo + B]), f"outputs differ at B={B}, sequences {lo}.."
    for s in (0, 17, 63):
        gi, go = decode_call(x, s, s + 1, n_kv)
        assert np.array_equal(gi, ref_idx[s:s + 1]) and np.array_equal(go, ref_out[s:s + 1]), f"B=1, seq {s}"
    # the bytes are real results: sequence 5 against the oracle
    q, k, w, qa, kv = (t[5].cpu() for t in x)
    p = np.array([n_kv - 1], np.int64)
    r_s, r_idx = oracle.score_select(bits(q), w.numpy(), bits(k), p, TOPK)
    check_index_sets(ref_idx[5, 0], r_idx[0], r_s[0, :n_kv], TOPK, "seq 5")
    K = bits(kv)
    o = oracle.attn(bits(qa), K, (K, DV), ref_idx[5], DQK ** -0.5)
    assert np.abs(bf16_to_f64(ref_out[5]) - bf16_to_f64(o)).max() <= ATTN_ATOL


def prefill_call(q, k, w, qa, kv, q0, rows, T_kv):
    """Indexer + attention for query rows q0 .. q0+rows-1 (positions), one call."""
    r0 = q0 - (T_kv - q.shape[1])
    qs, ws_, qas = q[:, r0:r0 + rows], w[:, r0:r0 + rows], qa[:, r0:r0 + rows]
    d = lcsi.indexer_desc(qs, k, ws_, TOPK, q0, T_kv=q0 + rows)
    ws = torch.empty(lcsi.idx_score_topk_ws_bytes(d) // 4 + 1, dtype=torch.float32, device="cuda")
    idx = torch.full((1, rows, TOPK), -9, dtype=torch.int32, device="cuda")
    lcsi.idx_score_topk(d, idx, ws)
    out = torch.full((1, rows, H_Q, DV), float("nan"), dtype=torch.bfloat16, device="cuda")
    a = lcsi.attn_desc(qas, kv, kv[..., :DV], out, TOPK, q0, DQK ** -0.5, T_kv=q0 + rows)
    lcsi.sparse_attn(a, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), bits(out)


@pytest.mark.parametrize("split", [1, 700, 2048])
def test_prefill_is_chunking_independent(split):
    """Rows 20000 .. 22999 against 23000 keys: the fused candidate pass
    (rows past its 16384 slots), one chunk versus chunks of `split` rows."""
    T_kv, rows = 23000, 3000
    q0 = T_kv - rows
    log(f"[determinism] prefill: rows {q0}..{T_kv - 1}, chunks of {split}")
    g = torch.Generator(device="cuda").manual_seed(12)
    q = torch.randn(1, rows, H_I, D_I, generator=g, device="cuda").div_(8).to(torch.bfloat16)
    k = torch.randn(1, T_kv, D_I, generator=g, device="cuda").div_(8).to(torch.bfloat16)
    w = torch.rand(1, rows, H_I, generator=g, device="cuda")
    qa = torch.randn(1, rows, H_Q, DQK, generator=g, device="cuda").to(torch.bfloat16)
    kv = torch.randn(1, T_kv, DQK, generator=g, device="cuda").to(torch.bfloat16)
    ref_idx, ref_out = prefill_call(q, k, w, qa, kv, q0, rows, T_kv)
    if split == 1:
        again_idx, again_out = prefill_call(q, k, w, qa, kv, q0, rows, T_kv)
        assert np.array_equal(again_idx, ref_idx) and np.array_equal(again_out, ref_out), "run to run"
        # the bytes are real results: a few rows against the oracle
        sample = [0, 1777, rows - 1]
        pos = np.array([q0 + t for t in sample], np.int64)
        r_s, r_idx = oracle.score_select(bits(q[0, sample]), w[0, sample].cpu().numpy(), bits(k[0]), pos, TOPK)
        for i, t in enumerate(sample):
            check_index_sets(ref_idx[0, t], r_idx[i], r_s[i, :pos[i] + 1], TOPK, f"row {t}")
        K = bits(kv[0])
        o = oracle.attn(bits(qa[0, sample]), K, (K, DV), ref_idx[0, sample], DQK ** -0.5)
        assert np.abs(bf16_to_f64(ref_out[0, sample]) - bf16_to_f64(o)).max() <= ATTN_ATOL
        return
    for c in range(0, rows, split):
        n = min(split, rows - c)
        if n < 2:
            continue    # (a one-row call is a decode call: its own arithmetic)
        gi, go = prefill_call(q, k, w, qa, kv, q0 + c, n, T_kv)
        assert np.array_equal(gi[0], ref_idx[0, c:c + n]), f"indices differ in the chunk at row {c}"
        assert np.array_equal(go[0], ref_out[0, c:c + n]), f"outputs differ in the chunk at row {c}"
