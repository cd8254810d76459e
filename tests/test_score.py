"""GPU indexer scores and end-to-end indices against the oracle.

Integer-exact mode (q, k integers in [-8, 8], w powers of two) makes every
score an exactly representable fp32 value whatever the summation order, so
GPU scores must equal the oracle's bit for bit and the indices must match
exactly.  Gaussian inputs are checked at the 1e-2 score tolerance and the
near-tie rule for index sets.  Both score kernels (the LDS-staged prefill
kernel and the split-key kernel used for few rows) and the three operand
formats (bf16 keys; fp8 e4m3 keys + scale widened to bf16; fp8 keys and fp8
queries + per-(token, head) scale on fp8 MFMA) are covered, with ragged
tails."""
import dataclasses

import zlib

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_idx_amd import inputs, lcsi
from helpers import bits, bytes_u8, check_index_sets, check_scores, log

pytestmark = pytest.mark.gpu


def gpu_indexer(q, k, w, top_k, q_pos0, k_scale=None, q_scale=None):
    """Returns (scores [B, T_q, ld] float32 host, idx [B, T_q, k] host).

    idx comes from the default call (the fused candidate pass wherever it
    applies) and must equal, bit for bit, the indices of the unfused call
    (every score row written, then selected), whose rows are the scores."""
    B, T_q = q.shape[:2]
    T_kv = k.shape[1]
    d = lcsi.indexer_desc(q, k, w, top_k, q_pos0, k_scale=k_scale, q_scale=q_scale)
    ws = torch.empty(lcsi.idx_score_topk_ws_bytes(d) // 4, dtype=torch.float32, device="cuda")
    idx = torch.empty((B, T_q, top_k), dtype=torch.int32, device="cuda")
    idx_u = torch.empty_like(idx)
    fused = lcsi.idx_score_topk_ws_bytes(d) > lcsi.idx_score_topk_ws_bytes(d, lcsi.LCSI_UNFUSED)
    log(f"  fused candidate pass: {fused}")
    lcsi.idx_score_topk(d, idx, ws)
    lcsi.idx_score_topk(d, idx_u, ws, flags=lcsi.LCSI_UNFUSED)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_u), "fused and unfused indices differ"
    ld = lcsi.score_ld(T_kv)
    return ws[:B * T_q * ld].view(B, T_q, ld).cpu().numpy(), idx.cpu().numpy()


def int_inputs(B, T_q, T_kv, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-8, 9, (B, T_q, H, D), generator=g).to(torch.float32)
    k = torch.randint(-8, 9, (B, T_kv, D), generator=g).to(torch.float32)
    w = (2.0 ** torch.randint(-3, 1, (B, T_q, H), generator=g)).to(torch.float32)
    return q, k, w


FORMATS = ["bf16", "k8", "qk8"]  # bf16 q/k; fp8 keys; fp8 keys and queries


def encode(fmt, q, k, B, T_q, T_kv, H, g):
    """Device operands and host copies in the format under test.  fp8 scales
    are powers of two, so integer inputs stay exact."""
    out = {}
    if fmt == "bf16":
        out["k"] = k.to(torch.bfloat16)
        out["k_scale"] = None
    else:
        out["k"] = k.to(torch.float8_e4m3fn).view(torch.uint8)  # integers |x| <= 8 are exact in e4m3
        out["k_scale"] = (2.0 ** torch.randint(-2, 2, (B, T_kv), generator=g)).to(torch.float32)
    if fmt == "qk8":
        out["q"] = q.to(torch.float8_e4m3fn).view(torch.uint8)
        out["q_scale"] = (2.0 ** torch.randint(-2, 2, (B, T_q, H), generator=g)).to(torch.float32)
    else:
        out["q"] = q.to(torch.bfloat16)
        out["q_scale"] = None
    return out


def host_q(x, b, rows):
    """(q rows for the oracle, their scales or None)."""
    if x["q"].dtype == torch.uint8:
        return bytes_u8(x["q"][b, rows]), x["q_scale"][b, rows].numpy()
    return bits(x["q"][b, rows]), None


def host_k(x, b):
    return bytes_u8(x["k"][b]) if x["k"].dtype == torch.uint8 else bits(x["k"][b])


def dev(x, name):
    return x[name].cuda() if x.get(name) is not None else None


SHAPES = [
    # B, T_q, T_kv, q_pos0, H, D, k         kernel the library picks
    (1, 300, 300, 0, 4, 64, 64),           # prefill (LDS-staged), causal from 0
    (1, 2048, 4100, 2052, 64, 128, 256),   # prefill, offset chunk, ragged key tail
    (1, 2048, 18000, 15952, 64, 128, 256),  # prefill, rows past 16384 keys: fused candidate pass
    (1, 130, 1000, 870, 16, 128, 100),     # prefill, H=16
    (3, 1, 9001, 9000, 64, 128, 2048),     # decode rows: split-key
    (2, 3, 8192, 8189, 8, 64, 512),        # few rows: split-key, H=8, D=64
    (1, 2, 6000, 5998, 32, 128, 128),      # few rows: split-key, H=32
]


def check_rows(T_q):
    """Rows checked against the oracle: both ends and a spread in between."""
    r = {0, 1, T_q - 2, T_q - 1} | set(np.linspace(0, T_q - 1, 10).astype(int).tolist())
    return sorted(x for x in r if 0 <= x < T_q)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
def test_score_integer_exact(shape, fmt):
    B, T_q, T_kv, q_pos0, H, D, k = shape
    log(f"[score-int] shape={shape} fmt={fmt}")
    seed = zlib.crc32(repr(shape).encode()) % 1000 + FORMATS.index(fmt)
    qf, kf, w = int_inputs(B, T_q, T_kv, H, D, seed=seed)
    x = encode(fmt, qf, kf, B, T_q, T_kv, H, torch.Generator().manual_seed(seed + 7))
    S, idx = gpu_indexer(dev(x, "q"), dev(x, "k"), w.cuda(), k, q_pos0, k_scale=dev(x, "k_scale"),
                         q_scale=dev(x, "q_scale"))
    rows = check_rows(T_q)
    pos = np.array([q_pos0 + t for t in rows])
    for b in range(B):
        hq, hqs = host_q(x, b, rows)
        rS, ridx = oracle.score_select(hq, w[b, rows].numpy(), host_k(x, b), pos, k,
                                       k_scale=x["k_scale"][b].numpy() if x["k_scale"] is not None else None,
                                       q_scale=hqs)
        for i, t in enumerate(rows):
            n = q_pos0 + t + 1
            assert np.array_equal(S[b, t, :n], rS[i, :n]), f"b={b} t={t}: scores differ"
            assert np.array_equal(idx[b, t], ridx[i]), f"b={b} t={t}: indices differ"


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
def test_score_gaussian(shape, fmt):
    B, T_q, T_kv, q_pos0, H, D, k = shape
    log(f"[score-gauss] shape={shape} fmt={fmt}")
    base = inputs.WORKLOADS[{"bf16": "prefill200k", "k8": "prefill1m", "qk8": "prefill1m_q8"}[fmt]]
    wl = dataclasses.replace(base, name=f"t{shape}", B=B, T_q=T_q, n_q=T_q, q_pos0=q_pos0,
                             T_kv=T_kv, H_I=H, D_I=D, top_k=k)
    x = inputs.indexer_inputs(wl, 0, "cpu")
    S, idx = gpu_indexer(dev(x, "q"), dev(x, "k"), dev(x, "w"), k, q_pos0, k_scale=dev(x, "k_scale"),
                         q_scale=dev(x, "q_scale"))
    rows = check_rows(T_q)
    pos = np.array([q_pos0 + t for t in rows])
    swaps = 0
    for b in range(B):
        hq, hqs = host_q(x, b, rows)
        rS, ridx = oracle.score_select(hq, x["w"][b, rows].numpy(), host_k(x, b), pos, k,
                                       k_scale=x["k_scale"][b].numpy() if x["k_scale"] is not None else None,
                                       q_scale=hqs)
        for i, t in enumerate(rows):
            n = q_pos0 + t + 1
            check_scores(S[b, t, :n], rS[i, :n], f"b={b} t={t}")
            swaps += check_index_sets(idx[b, t], ridx[i], rS[i, :n], k, f"b={b} t={t}")
    log(f"  near-tie swaps: {swaps}")


def test_score_weight_scaling_and_h1_identity():
    """Scaling w by 2 doubles every GPU score exactly and keeps the indices."""
    B, T_q, T_kv, q_pos0, H, D, k = 1, 40, 3000, 2960, 64, 128, 300
    g = torch.Generator().manual_seed(5)
    q = (torch.randn(B, T_q, H, D, generator=g) / 8).to(torch.bfloat16).cuda()
    kk = (torch.randn(B, T_kv, D, generator=g) / 8).to(torch.bfloat16).cuda()
    w = torch.rand(B, T_q, H, generator=g).cuda()
    S1, i1 = gpu_indexer(q, kk, w, k, q_pos0)
    S2, i2 = gpu_indexer(q, kk, 2 * w, k, q_pos0)
    for t in range(T_q):
        n = q_pos0 + t + 1
        assert np.array_equal(S2[0, t, :n], 2 * S1[0, t, :n])
    assert np.array_equal(i1, i2)


@pytest.mark.parametrize("T_kv", [6000, 20000])
@pytest.mark.parametrize("fmt", FORMATS)
def test_prefill_and_splitkey_kernels_agree_bitwise(fmt, T_kv):
    """The same rows scored as one batch of many rows (prefill kernel; with
    20000 keys through the fused candidate pass) and as single-row calls
    (split-key kernel) give identical bits: chunking never changes a score
    or an index."""
    H, D, k = 64, 128, 512
    T_q, q_pos0 = 2048, T_kv - 2048   # 256 workgroups: the prefill kernel
    base = inputs.WORKLOADS[{"bf16": "prefill200k", "k8": "prefill1m", "qk8": "prefill1m_q8"}[fmt]]
    wl = dataclasses.replace(base, name="agree", B=1, T_q=T_q, n_q=T_q, q_pos0=q_pos0, T_kv=T_kv,
                             H_I=H, D_I=D, top_k=k)
    x = {n: (v.cuda() if v is not None else None) for n, v in inputs.indexer_inputs(wl, 0, "cpu").items()}
    S_all, i_all = gpu_indexer(x["q"], x["k"], x["w"], k, q_pos0, k_scale=x["k_scale"], q_scale=x["q_scale"])
    for t in (0, 17, 1000, 2047):
        qs = x["q_scale"][:, t:t + 1] if x["q_scale"] is not None else None
        S1, i1 = gpu_indexer(x["q"][:, t:t + 1], x["k"], x["w"][:, t:t + 1], k, q_pos0 + t,
                             k_scale=x["k_scale"], q_scale=qs)
        n = q_pos0 + t + 1
        assert np.array_equal(S1[0, 0, :n], S_all[0, t, :n])
        assert np.array_equal(i1[0, 0], i_all[0, t])


@pytest.mark.parametrize("shape", [(3, 1, 9001, 9000, 2048),      # decode rows: split-key kernel
                                   (1, 512, 4100, 3588, 256)])     # prefill kernel
@pytest.mark.parametrize("fmt", FORMATS)
def test_padded_key_rows_score_like_packed_rows(fmt, shape):
    """Keys whose rows sit in a wider buffer (row stride D + 48 bytes' worth
    of elements, the padding filled with 0x7F bytes: a huge bf16 value, an
    fp8 NaN) score and select bit for bit like the same keys packed: every
    kernel reads a key row's D elements and nothing past them."""
    B, T_q, T_kv, q_pos0, k = shape
    H, D = 64, 128
    log(f"[score-padded] shape={shape} fmt={fmt}")
    base = inputs.WORKLOADS[{"bf16": "prefill200k", "k8": "prefill1m", "qk8": "prefill1m_q8"}[fmt]]
    wl = dataclasses.replace(base, name="padded", B=B, T_q=T_q, n_q=T_q, q_pos0=q_pos0, T_kv=T_kv,
                             H_I=H, D_I=D, top_k=k)
    x = {n: (v.cuda() if v is not None else None) for n, v in inputs.indexer_inputs(wl, 0, "cpu").items()}
    S_p, i_p = gpu_indexer(x["q"], x["k"], x["w"], k, q_pos0, k_scale=x["k_scale"], q_scale=x["q_scale"])
    pad = 48 // x["k"].element_size()
    if x["k"].element_size() == 1:
        wide = torch.full((B, T_kv, D + pad), 0x7F, dtype=torch.uint8, device="cuda").view(x["k"].dtype)
    else:
        wide = torch.full((B, T_kv, D + pad), 0x7F7F, dtype=torch.int16, device="cuda").view(x["k"].dtype)
    wide[..., :D] = x["k"]
    kv = wide[..., :D]
    assert kv.stride(1) == D + pad
    S_w, i_w = gpu_indexer(x["q"], kv, x["w"], k, q_pos0, k_scale=x["k_scale"], q_scale=x["q_scale"])
    for t in range(T_q):
        n = q_pos0 + t + 1
        assert np.array_equal(S_w[:, t, :n], S_p[:, t, :n]), f"t={t}: scores differ"
    assert np.array_equal(i_w, i_p)


@pytest.mark.parametrize("fmt", FORMATS)
def test_degenerate_rows(fmt):
    """One key (T_kv = 1) and very short causal rows mixing n <= k and n > k:
    scores and indices as the oracle's, -1 padding after the n entries."""
    for (T_q, T_kv, q_pos0, k) in [(1, 1, 0, 2048), (3, 3, 0, 2), (5, 7, 2, 1)]:
        H, D = 64, 128
        base = inputs.WORKLOADS[{"bf16": "prefill200k", "k8": "prefill1m", "qk8": "prefill1m_q8"}[fmt]]
        wl = dataclasses.replace(base, name=f"deg{T_q}_{T_kv}", B=1, T_q=T_q, n_q=T_q, q_pos0=q_pos0,
                                 T_kv=T_kv, H_I=H, D_I=D, top_k=k)
        x = inputs.indexer_inputs(wl, 0, "cpu")
        S, idx = gpu_indexer(dev(x, "q"), dev(x, "k"), dev(x, "w"), k, q_pos0, k_scale=dev(x, "k_scale"),
                             q_scale=dev(x, "q_scale"))
        rows = list(range(T_q))
        hq, hqs = host_q(x, 0, rows)
        pos = np.array([q_pos0 + t for t in rows])
        rS, ridx = oracle.score_select(hq, x["w"][0, rows].numpy(), host_k(x, 0), pos, k,
                                       k_scale=x["k_scale"][0].numpy() if x["k_scale"] is not None else None,
                                       q_scale=hqs)
        for t in rows:
            n = q_pos0 + t + 1
            check_scores(S[0, t, :n], rS[t, :n], f"T_kv={T_kv} t={t}")
            assert np.array_equal(idx[0, t], ridx[t]), f"T_kv={T_kv} t={t}: {idx[0, t][:8]} vs {ridx[t][:8]}"
            assert (idx[0, t, min(n, k):] == -1).all()


def test_fp8_keys_widen_exactly_for_every_finite_code():
    """The fp8-key path widens e4m3 keys to bf16 with the hardware conversion
    at scale 1: exact for every finite code.  Key s holds code s in its first
    element (the two NaN codes replaced by zero), one head reads it with +1
    and another row with -1, so the scores are ReLU(+-value) bit for bit."""
    codes = np.array([c if (c & 0x7F) != 0x7F else 0 for c in range(256)], np.uint8)
    T_kv, T_q, H, D = 256, 2, 4, 64
    k = torch.zeros((1, T_kv, D), dtype=torch.uint8)
    k[0, :, 0] = torch.from_numpy(codes)
    q = torch.zeros((1, T_q, H, D), dtype=torch.float32)
    q[0, 0, 0, 0], q[0, 1, 0, 0] = 1.0, -1.0
    w = torch.zeros((1, T_q, H), dtype=torch.float32)
    w[0, :, 0] = 1.0
    ks = torch.ones((1, T_kv), dtype=torch.float32)
    S, _ = gpu_indexer(q.to(torch.bfloat16).cuda(), k.cuda(), w.cuda(), 8, T_kv - T_q, k_scale=ks.cuda())
    val = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    n0 = T_kv - 1  # row 0 sees keys 0 .. 254
    want0 = (np.maximum(val[:n0], 0) + 0.0).astype(np.float32)   # (+0.0 folds a -0)
    want1 = (np.maximum(-val, 0) + 0.0).astype(np.float32)
    assert np.array_equal(S[0, 0, :n0].view(np.uint32), want0.view(np.uint32))
    assert np.array_equal(S[0, 1, :T_kv].view(np.uint32), want1.view(np.uint32))
