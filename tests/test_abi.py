"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/lcsi.h declares, and rejects every bad argument with
its status code before anything is launched.  Pointers here are fake but
aligned addresses: validation only looks at NULL-ness and alignment, and
every call below either fails validation or runs in query mode, so nothing
is ever dereferenced or launched."""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

from long_context_sparse_idx_amd import lcsi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcsi.h")
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}()]*(?:\([^)]*\)[^;{}()]*)*\)\s*;", text)
    return sorted(set(names))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("idx_score_topk", "sparse_attn", "run_layer_group"):
        assert n in names
    assert set(names) == set(lcsi.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", lcsi._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lcsi.lib, name)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lcsi.strerror(code)
    assert lcsi.strerror(-99) == "unknown status"


def test_score_ld():
    assert lcsi.score_ld(1) == 64
    assert lcsi.score_ld(64) == 64
    assert lcsi.score_ld(200000) == 200000
    assert lcsi.score_ld(131073) == 131136


# ---------------------------------------------------------------- indexer

def good_indexer(**over):
    d = lcsi.Indexer()
    d.B, d.T_q, d.T_kv, d.H_I, d.D_I, d.top_k = 2, 16, 100, 64, 128, 8
    d.key_dtype = lcsi.LCSI_KEY_BF16
    d.q_pos0 = 84
    d.q, d.q_sb, d.q_st, d.q_sh = FAKE, 16 * 64 * 128, 64 * 128, 128
    d.k, d.k_sb, d.k_st = FAKE, 100 * 128, 128
    d.w, d.w_sb, d.w_st = FAKE, 16 * 64, 64
    for k, v in over.items():
        setattr(d, k, v)
    return d


def call_idx(d, idx=FAKE, ws=None, nbytes=None, flags=0, sb=16 * 8, st=8):
    n = ctypes.c_size_t(nbytes if nbytes is not None else 0)
    ref = ctypes.byref(n) if nbytes is not None or ws is None else None
    rc = lcsi.lib.idx_score_topk(ctypes.byref(d), ctypes.c_void_p(idx), sb, st,
                                 ctypes.c_void_p(ws) if ws else None, ref, flags, None)
    return rc, n.value


def test_indexer_query_mode_returns_workspace_size():
    rows_bytes = 2 * 16 * lcsi.score_ld(100) * 4
    # short rows (at most 16384 keys): score rows only
    rc, n = call_idx(good_indexer())
    assert rc == 0 and n == rows_bytes
    # the fused pass (H_I >= 16, prefill kernel, a row longer than 16384
    # keys) adds 256-aligned counts, the 256-aligned list of unsettled rows
    # (a count and 64 row ids) and 16384 candidate pairs per row
    # (1024 queries: enough workgroups for the prefill kernel)
    long_rows = dict(T_q=1024, T_kv=20000, q_pos0=18976, q_sb=1024 * 64 * 128, k_sb=20000 * 128,
                     w_sb=1024 * 64)
    long_bytes = 2 * 1024 * lcsi.score_ld(20000) * 4
    rc, n = call_idx(good_indexer(**long_rows), sb=1024 * 8)
    assert rc == 0
    assert n == long_bytes + 2 * 1024 * 4 + 512 + 2 * 1024 * 16384 * 8
    for flags in (lcsi.LCSI_UNFUSED, lcsi.LCSI_SCORES_ONLY, lcsi.LCSI_SCORES_PRESET):
        rc, n = call_idx(good_indexer(**long_rows), sb=1024 * 8, flags=flags)
        assert rc == 0 and n == long_bytes, flags
    # no fused pass below 16 heads
    h8 = dict(long_rows, H_I=8, q_sb=1024 * 8 * 128, q_st=8 * 128, w_sb=1024 * 8, w_st=8)
    rc, n = call_idx(good_indexer(**h8), sb=1024 * 8)
    assert rc == 0 and n == long_bytes
    rc, n = call_idx(good_indexer(key_dtype=lcsi.LCSI_KEY_FP8_E4M3, k_scale=FAKE, ks_sb=100,
                                  k_sb=100 * 128, k_st=128))
    assert rc == 0 and n > 0


@pytest.mark.parametrize("last_row_keys,fused", [(16384, False), (16385, True)])
def test_fused_pass_needs_a_row_longer_than_the_slots(last_row_keys, fused):
    """The fused pass is planned only when the longest row (q_pos0 + T_q
    causal keys) exceeds the 16384 candidate slots of a row, and with enough
    rows for the prefill kernel (2 x 1024 queries at 64 heads)."""
    T_q, T_kv = 1024, last_row_keys
    d = dict(T_q=T_q, T_kv=T_kv, q_pos0=T_kv - T_q, q_sb=T_q * 64 * 128, k_sb=T_kv * 128, w_sb=T_q * 64)
    rc, n = call_idx(good_indexer(**d), sb=T_q * 8)
    rc_u, n_u = call_idx(good_indexer(**d), sb=T_q * 8, flags=lcsi.LCSI_UNFUSED)
    assert rc == 0 and rc_u == 0
    assert n_u == 2 * T_q * lcsi.score_ld(T_kv) * 4
    assert (n > n_u) == fused
    # fewer rows (the split-key kernel scores them): never fused
    rc, n = call_idx(good_indexer(**dict(d, B=1)), sb=T_q * 8)
    assert rc == 0 and n == n_u // 2


def test_noalloc_refuses_calls_beyond_its_scratch():
    """Checked on the host before anything is launched: a decode call whose
    partials exceed the static scratch returns LCSI_ESCRATCH; bad
    descriptors fail as for sparse_attn."""
    big = good_attn(B=128, T_q=1, H_q=64, q_pos0=99, top_k=2048)  # 128 * 8 * 64 * 1 KB > 48 MiB
    rc = lcsi.lib.sparse_attn_noalloc(ctypes.byref(big), ctypes.c_void_p(FAKE), 2048, 2048, None)
    assert rc == lcsi.LCSI_ESCRATCH
    assert "scratch" in lcsi.strerror(rc)
    bad = good_attn(T_q=1, q_pos0=99, top_k=0)
    assert lcsi.lib.sparse_attn_noalloc(ctypes.byref(bad), ctypes.c_void_p(FAKE), 8, 8, None) == lcsi.LCSI_EINVAL
    ok = good_attn(T_q=1, q_pos0=99, top_k=2048)
    assert lcsi.lib.sparse_attn_noalloc(ctypes.byref(ok), None, 8, 8, None) == lcsi.LCSI_EINVAL
    assert lcsi.lib.sparse_attn_noalloc(None, ctypes.c_void_p(FAKE), 8, 8, None) == lcsi.LCSI_EINVAL


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, lcsi.LCSI_EINVAL),
    ("T_q", 0, lcsi.LCSI_EINVAL),
    ("T_kv", 0, lcsi.LCSI_EINVAL),
    ("q_pos0", -1, lcsi.LCSI_EINVAL),
    ("q_pos0", 85, lcsi.LCSI_EINVAL),          # q_pos0 + T_q > T_kv
    ("top_k", 0, lcsi.LCSI_EINVAL),
    ("top_k", 2049, lcsi.LCSI_EUNSUPPORTED),
    ("H_I", 0, lcsi.LCSI_EINVAL),
    ("H_I", 12, lcsi.LCSI_EUNSUPPORTED),
    ("H_I", 128, lcsi.LCSI_EUNSUPPORTED),
    ("D_I", 96, lcsi.LCSI_EUNSUPPORTED),
    ("key_dtype", 7, lcsi.LCSI_EINVAL),
    ("q", 0, lcsi.LCSI_EINVAL),
    ("k", 0, lcsi.LCSI_EINVAL),
    ("w", 0, lcsi.LCSI_EINVAL),
    ("q", FAKE + 8, lcsi.LCSI_EALIGN),
    ("k", FAKE + 2, lcsi.LCSI_EALIGN),
    ("w", FAKE + 4, lcsi.LCSI_EALIGN),
    ("q_sh", 132, lcsi.LCSI_EALIGN),
    ("k_st", 130, lcsi.LCSI_EALIGN),
    ("w_st", 66, lcsi.LCSI_EALIGN),
    ("q_st", -8, lcsi.LCSI_EINVAL),
])
def test_indexer_rejects_bad_fields(field, value, code):
    rc, _ = call_idx(good_indexer(**{field: value}))
    assert rc == code


def test_indexer_fp8_needs_scale_and_16_byte_rows():
    d = good_indexer(key_dtype=lcsi.LCSI_KEY_FP8_E4M3)
    assert call_idx(d)[0] == lcsi.LCSI_EINVAL                 # no k_scale
    d = good_indexer(key_dtype=lcsi.LCSI_KEY_FP8_E4M3, k_scale=FAKE + 2, ks_sb=100)
    assert call_idx(d)[0] == lcsi.LCSI_EALIGN
    d = good_indexer(key_dtype=lcsi.LCSI_KEY_FP8_E4M3, k_scale=FAKE, ks_sb=100, k_st=136)
    assert call_idx(d)[0] == lcsi.LCSI_EALIGN                 # 136 B rows


def test_indexer_envelope_limits():
    # the score rows of one workgroup (512 / H_I rows) must stay below 2 GiB
    big = (1 << 31) // (4 * 512 // 4) + 64          # H_I = 4: 128 rows
    assert call_idx(good_indexer(H_I=4, T_kv=big, q_pos0=big - 16, k_sb=big * 128))[0] == lcsi.LCSI_EUNSUPPORTED
    assert call_idx(good_indexer(H_I=64, T_kv=big, q_pos0=big - 16, k_sb=big * 128))[0] == 0
    # a 128-key tile of keys is addressed with 32-bit offsets: key rows below 16 MiB
    assert call_idx(good_indexer(k_st=(1 << 23), k_sb=100 * (1 << 23)))[0] == lcsi.LCSI_EUNSUPPORTED
    assert call_idx(good_indexer(k_st=(1 << 23) - 8, k_sb=100 * ((1 << 23) - 8)))[0] == 0


def test_indexer_fp8_queries_rules():
    fp8k = dict(key_dtype=lcsi.LCSI_KEY_FP8_E4M3, k_scale=FAKE, ks_sb=100)
    q8 = dict(q_dtype=lcsi.LCSI_Q_FP8_E4M3, q_scale=FAKE, qs_sb=16 * 64, qs_st=64)
    assert call_idx(good_indexer(**fp8k, **q8))[0] == 0
    assert call_idx(good_indexer(**fp8k, **{**q8, "q_dtype": 5}))[0] == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(**q8))[0] == lcsi.LCSI_EUNSUPPORTED            # fp8 queries need fp8 keys
    assert call_idx(good_indexer(**fp8k, **{**q8, "q_scale": 0}))[0] == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(**fp8k, **{**q8, "q_scale": FAKE + 2}))[0] == lcsi.LCSI_EALIGN
    assert call_idx(good_indexer(**fp8k, **{**q8, "qs_st": -1}))[0] == lcsi.LCSI_EINVAL
    # fp8 query rows: strides in bytes, multiples of 16
    assert call_idx(good_indexer(**fp8k, **q8, q_sh=136))[0] == lcsi.LCSI_EALIGN
    assert call_idx(good_indexer(**fp8k, **q8, q_sh=144))[0] == 0


def test_indexer_output_and_flags():
    need = call_idx(good_indexer())[1]
    # output checks apply when a workspace is given (not in query mode)
    assert call_idx(good_indexer(), idx=0, ws=FAKE, nbytes=need)[0] == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(), idx=FAKE + 2, ws=FAKE, nbytes=need)[0] == lcsi.LCSI_EALIGN
    assert call_idx(good_indexer(), st=-1, ws=FAKE, nbytes=need)[0] == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(), flags=3)[0] == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(), flags=8)[0] == lcsi.LCSI_EINVAL
    # query mode needs only the descriptor
    assert call_idx(good_indexer(), idx=0) == (0, need)
    # scores-only needs no index output
    assert call_idx(good_indexer(), idx=0, flags=lcsi.LCSI_SCORES_ONLY)[0] == 0
    # preset mode reads only B, T_q, T_kv, q_pos0, top_k
    d = lcsi.preset_desc(2, 16, 100, 84, 8)
    rc, n = call_idx(d, flags=lcsi.LCSI_SCORES_PRESET)
    assert rc == 0 and n == 2 * 16 * 128 * 4


def test_indexer_workspace_rules():
    need = call_idx(good_indexer())[1]
    # no workspace and no size pointer: a workspace is always required
    rc = lcsi.lib.idx_score_topk(ctypes.byref(good_indexer()), ctypes.c_void_p(FAKE), 128, 8,
                                 None, None, 0, None)
    assert rc == lcsi.LCSI_EWORKSPACE
    # a workspace without its capacity
    rc = lcsi.lib.idx_score_topk(ctypes.byref(good_indexer()), ctypes.c_void_p(FAKE), 128, 8,
                                 ctypes.c_void_p(FAKE), None, 0, None)
    assert rc == lcsi.LCSI_EINVAL
    assert call_idx(good_indexer(), ws=FAKE, nbytes=need - 1)[0] == lcsi.LCSI_EWORKSPACE
    assert call_idx(good_indexer(), ws=FAKE + 128, nbytes=need)[0] == lcsi.LCSI_EALIGN


# -------------------------------------------------------------- attention

def good_attn(**over):
    d = lcsi.Attn()
    d.B, d.T_q, d.T_kv, d.H_q, d.D_qk, d.D_v, d.top_k = 2, 16, 100, 32, 576, 512, 8
    d.sm_scale = 0.04
    d.q_pos0 = 84
    d.q, d.q_sb, d.q_st, d.q_sh = FAKE, 16 * 32 * 576, 32 * 576, 576
    d.k, d.k_sb, d.k_st = FAKE, 100 * 576, 576
    d.v, d.v_sb, d.v_st = FAKE, 100 * 576, 576
    d.out, d.o_sb, d.o_st, d.o_sh = FAKE, 16 * 32 * 512, 32 * 512, 512
    for k, v in over.items():
        setattr(d, k, v)
    return d


def call_attn(d, idx=FAKE, query=True):
    n = ctypes.c_size_t(0)
    return lcsi.lib.sparse_attn(ctypes.byref(d), ctypes.c_void_p(idx), 128, 8, None,
                                ctypes.byref(n) if query else None, None), n.value


def test_attn_query_mode():
    # a decode call (one query row per sequence) with long lists: partials of
    # ceil(top_k / 256) parts per row, whatever the batch size
    for B in (1, 2, 32, 300):
        rc, n = call_attn(good_attn(B=B, T_q=1, q_pos0=99, top_k=2048))
        parts, H, Dv = 8, 32, 512
        po = (B * parts * H * Dv * 2 + 255) // 256 * 256
        assert rc == 0 and n == po + B * parts * H * 8, (B, n)
    rc, n = call_attn(good_attn(B=2, T_q=1, q_pos0=99, top_k=256))
    assert rc == 0 and n == 0           # one part: no partials
    # multi-row calls never split, however few rows they hold
    for B, T_q in ((2, 16), (1, 2), (1, 1024)):
        rc, n = call_attn(good_attn(B=B, T_q=T_q, q_pos0=0, T_kv=1024, top_k=2048))
        assert rc == 0 and n == 0, (B, T_q)
    # a workspace-free call is refused when partials are needed
    assert call_attn(good_attn(T_q=1, q_pos0=99, top_k=2048), query=False)[0] == lcsi.LCSI_EWORKSPACE


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, lcsi.LCSI_EINVAL),
    ("q_pos0", 90, lcsi.LCSI_EINVAL),
    ("top_k", 0, lcsi.LCSI_EINVAL),
    ("top_k", 4096, lcsi.LCSI_EUNSUPPORTED),
    ("H_q", 0, lcsi.LCSI_EINVAL),
    ("H_q", 65, lcsi.LCSI_EUNSUPPORTED),
    ("D_qk", 192, lcsi.LCSI_EUNSUPPORTED),
    ("D_v", 128, lcsi.LCSI_EUNSUPPORTED),
    ("sm_scale", float("inf"), lcsi.LCSI_EINVAL),
    ("sm_scale", float("nan"), lcsi.LCSI_EINVAL),
    ("sm_scale", 0.0, lcsi.LCSI_EINVAL),
    ("sm_scale", -0.04, lcsi.LCSI_EINVAL),
    ("q", 0, lcsi.LCSI_EINVAL),
    ("out", 0, lcsi.LCSI_EINVAL),
    ("v", FAKE + 2, lcsi.LCSI_EALIGN),
    ("k_st", 580, lcsi.LCSI_EALIGN),
    ("o_sh", 516, lcsi.LCSI_EALIGN),
    ("k_st", 1 << 31, lcsi.LCSI_EUNSUPPORTED),   # KV row stride of 4 GiB (bf16 elements)
    ("v_st", 1 << 31, lcsi.LCSI_EUNSUPPORTED),
])
def test_attn_rejects_bad_fields(field, value, code):
    assert call_attn(good_attn(**{field: value}))[0] == code


def test_attn_rejects_bad_index_pointer():
    # outside query mode (no workspace needed at top_k = 8): index checks apply
    assert call_attn(good_attn(), idx=0, query=False)[0] == lcsi.LCSI_EINVAL
    assert call_attn(good_attn(), idx=FAKE + 1, query=False)[0] == lcsi.LCSI_EALIGN
    # query mode needs only the descriptor
    assert call_attn(good_attn(), idx=0)[0] == 0


# ------------------------------------------------------------ layer group

def call_group(pattern, n_idx=None, idx_over=None, attn_over=None, n_slots=1, cache=FAKE, query=True):
    L = len(pattern)
    nf = sum(pattern) if n_idx is None else n_idx
    pat = (ctypes.c_uint8 * L)(*pattern)
    ia = (lcsi.Indexer * max(nf, 1))(*[good_indexer(**(idx_over or {})) for _ in range(max(nf, 1))])
    aa = (lcsi.Attn * L)(*[good_attn(**(attn_over or {})) for _ in range(L)])
    n = ctypes.c_size_t(0)
    if query:
        rc = lcsi.lib.run_layer_group(L, pat, ia, nf, aa, ctypes.c_void_p(cache), n_slots, 0, 128, 8,
                                      None, ctypes.byref(n), None, None)
    else:  # a workspace that is too small: fails before any launch
        n.value = 1
        rc = lcsi.lib.run_layer_group(L, pat, ia, nf, aa, ctypes.c_void_p(cache), n_slots, 0, 128, 8,
                                      ctypes.c_void_p(FAKE), ctypes.byref(n), None, None)
    return rc, n.value


def test_layer_group_query_and_pattern_errors():
    rc, n = call_group([1, 0, 0, 0])
    assert rc == 0 and n >= 2 * 16 * 128 * 4
    assert call_group([0, 1, 0, 0])[0] == lcsi.LCSI_EPATTERN     # leading S
    assert call_group([1, 0, 1, 0], n_idx=1)[0] == lcsi.LCSI_EPATTERN
    assert call_group([1, 0, 0, 0], n_idx=2)[0] == lcsi.LCSI_EPATTERN
    assert call_group([1, 0], n_slots=0)[0] == lcsi.LCSI_EINVAL
    assert call_group([1, 0], cache=0)[0] == 0                       # query: descriptors only
    assert call_group([1, 0], cache=0, query=False)[0] == lcsi.LCSI_EINVAL
    assert call_group([1, 0], cache=FAKE + 2, query=False)[0] == lcsi.LCSI_EALIGN
    assert call_group([1, 0], query=False)[0] == lcsi.LCSI_EWORKSPACE
    # descriptors of one group must agree on rows and top_k
    assert call_group([1, 0], attn_over={"top_k": 16})[0] == lcsi.LCSI_EINVAL
    assert call_group([1, 0], idx_over={"H_I": 48})[0] == lcsi.LCSI_EUNSUPPORTED
    assert call_group([1, 0], attn_over={"D_qk": 64})[0] == lcsi.LCSI_EUNSUPPORTED


def test_binding_checks_layouts_and_dtypes():
    """The descriptors carry strides for the outer dimensions only: the
    binding refuses tensors whose last dimension is not contiguous, and wrong
    dtypes or shapes, before anything reaches the library."""
    B, T, H, D = 1, 8, 16, 64
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    k = torch.zeros(B, T, D, dtype=torch.bfloat16)
    w = torch.zeros(B, T, H, dtype=torch.float32)
    d = lcsi.indexer_desc(q, k, w, 4, 0)
    assert (d.q_sb, d.q_st, d.q_sh, d.k_st, d.w_st) == (T * H * D, H * D, D, D, H)
    bad = [
        dict(q=torch.zeros(B, T, D, H, dtype=torch.bfloat16).transpose(2, 3)),
        dict(k=torch.zeros(B, D, T, dtype=torch.bfloat16).transpose(1, 2)),
        dict(w=w.double()),
        dict(q=q.float()),
        dict(w=torch.zeros(B, T, H + 1)),
        dict(k=torch.zeros(B, T, D, dtype=torch.uint8)),  # fp8 keys without k_scale
    ]
    for over in bad:
        args = dict(q=q, k=k, w=w)
        args.update(over)
        with pytest.raises(ValueError):
            lcsi.indexer_desc(args["q"], args["k"], args["w"], 4, 0)
    with pytest.raises(ValueError):  # fp8 queries without q_scale
        lcsi.indexer_desc(torch.zeros(B, T, H, D, dtype=torch.uint8), torch.zeros(B, T, D, dtype=torch.uint8),
                          w, 4, 0, k_scale=torch.ones(B, T))
    kv = torch.zeros(B, T, 576, dtype=torch.bfloat16)
    qa = torch.zeros(B, T, 4, 576, dtype=torch.bfloat16)
    out = torch.zeros(B, T, 4, 512, dtype=torch.bfloat16)
    a = lcsi.attn_desc(qa, kv, kv[..., :512], out, 4, 0, 0.1)
    assert (a.k_st, a.v_st, a.o_sh) == (576, 576, 512)
    with pytest.raises(ValueError):
        lcsi.attn_desc(qa, kv, kv[..., :512], torch.zeros(B, T, 512, 4, dtype=torch.bfloat16).transpose(2, 3),
                       4, 0, 0.1)
    with pytest.raises(ValueError):
        lcsi.attn_desc(qa.float(), kv, kv[..., :512], out, 4, 0, 0.1)
    # shapes that disagree with q would send the kernels past the buffers
    bad_attn = [
        dict(out=torch.zeros(B, T, 4, 128, dtype=torch.bfloat16)),          # Dv of out != Dv of v
        dict(out=torch.zeros(B, T + 1, 4, 512, dtype=torch.bfloat16)),      # T_q of out
        dict(out=torch.zeros(B, T, 8, 512, dtype=torch.bfloat16)),          # heads of out
        dict(k=torch.zeros(B, T, 128, dtype=torch.bfloat16)),               # Dqk of k != Dqk of q
        dict(k=torch.zeros(B + 1, T, 576, dtype=torch.bfloat16)),           # batch of k
        dict(v=torch.zeros(B, T - 1, 512, dtype=torch.bfloat16)),           # rows of v != rows of k
        dict(v=torch.zeros(B + 1, T, 512, dtype=torch.bfloat16)),           # batch of v
        dict(T_kv=T + 1),                                                   # more keys than k holds
        dict(T_kv=0),
    ]
    for over in bad_attn:
        args = dict(q=qa, k=kv, v=kv[..., :512], out=out, T_kv=None)
        args.update(over)
        with pytest.raises(ValueError):
            lcsi.attn_desc(args["q"], args["k"], args["v"], args["out"], 4, 0, 0.1, T_kv=args["T_kv"])
    # indexer: key prefix, scale shapes
    with pytest.raises(ValueError):
        lcsi.indexer_desc(q, k, w, 4, 0, T_kv=T + 1)
    k8 = torch.zeros(B, T, D, dtype=torch.uint8)
    q8 = torch.zeros(B, T, H, D, dtype=torch.uint8)
    with pytest.raises(ValueError):   # k_scale shorter than the keys
        lcsi.indexer_desc(q, k8, w, 4, 0, k_scale=torch.ones(B, T - 1))
    with pytest.raises(ValueError):   # q_scale of the wrong shape
        lcsi.indexer_desc(q8, k8, w, 4, 0, k_scale=torch.ones(B, T), q_scale=torch.ones(B, T, H + 1))
    d8 = lcsi.indexer_desc(q8, k8, w, 4, 0, k_scale=torch.ones(B, T), q_scale=torch.ones(B, T, H))
    assert d8.q_dtype == lcsi.LCSI_Q_FP8_E4M3 and d8.T_kv == T
    # index tensors: rows must match the descriptor, entries >= top_k
    for bad_idx in (torch.zeros(B, T, 3, dtype=torch.int32), torch.zeros(B, T + 1, 4, dtype=torch.int32),
                    torch.zeros(B + 1, T, 4, dtype=torch.int32), torch.zeros(B, T, 4, dtype=torch.int64),
                    torch.zeros(B, 4, T, dtype=torch.int32).transpose(1, 2)):
        with pytest.raises(ValueError):
            lcsi.sparse_attn(a, bad_idx)
        with pytest.raises(ValueError):
            lcsi.idx_score_topk(d, bad_idx, torch.zeros(16))
    with pytest.raises(ValueError):   # no indices and not scores-only
        lcsi.idx_score_topk(d, None, torch.zeros(16))
    # an index cache too small for its slots
    small = torch.zeros(2 * B * T * 4 - 1, dtype=torch.int32)
    with pytest.raises(ValueError):
        lcsi.run_layer_group([1, 0], [d], [a, a], small, 2, B * T * 4, T * 4, 4)
    with pytest.raises(ValueError):
        lcsi.idx_overlap(torch.zeros(B, T, 4, dtype=torch.int32), torch.zeros(B, T, 5, dtype=torch.int32))


def test_binding_refuses_to_load_without_the_library(tmp_path):
    """No fallback: a copy of the binding next to no built library raises
    ImportError on import instead of running anything else."""
    pkg = tmp_path / "pkg_no_lib"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    src = os.path.join(os.path.dirname(lcsi.__file__), "lcsi.py")
    (pkg / "lcsi.py").write_text(open(src).read())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import pkg_no_lib.lcsi\nexcept ImportError as e:\n    print('refused:', e)\n"
            "else:\n    print('loaded')\n") % str(tmp_path)
    env = {k: v for k, v in os.environ.items() if k != "LCSI_LIB"}
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("refused:") and "no fallback" in r.stdout, r.stdout
