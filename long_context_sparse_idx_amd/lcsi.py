"""Thin ctypes binding of liblcsi.so (the C ABI in include/lcsi.h).

Argument marshalling only: torch tensors become device pointers, element
strides and the current HIP stream; every step of the path runs in the
library's kernels.  Workspaces the caller does not pass are allocated here
as plain torch device tensors.  Any non-zero status raises ``LcsiError``.
The library must be built first (``python -m long_context_sparse_idx_amd.build``);
importing this module without it raises immediately -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

# LCSI_LIB names another build of the same library to load instead (the
# sanitizer test points it at a host-ASan build); never a fallback.
_LIB_PATH = os.environ.get("LCSI_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblcsi.so")

LCSI_OK = 0
LCSI_EINVAL = -1
LCSI_EUNSUPPORTED = -2
LCSI_EWORKSPACE = -3
LCSI_EPATTERN = -4
LCSI_EALIGN = -5
LCSI_EHIP = -6
LCSI_ESCRATCH = -7
LCSI_KEY_BF16 = 0
LCSI_KEY_FP8_E4M3 = 1
LCSI_Q_BF16 = 0
LCSI_Q_FP8_E4M3 = 1
LCSI_SCORES_PRESET = 1
LCSI_SCORES_ONLY = 2
LCSI_UNFUSED = 4
LCSI_MAX_TOPK = 2048
LCSI_NOALLOC_SCRATCH_BYTES = 48 << 20

EXPORTED = ("idx_score_topk", "sparse_attn", "sparse_attn_noalloc", "run_layer_group", "idx_overlap",
            "lcsi_score_ld", "lcsi_strerror")


class LcsiError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({strerror(code)})")


class Indexer(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T_q", ctypes.c_int32), ("T_kv", ctypes.c_int32),
                ("H_I", ctypes.c_int32), ("D_I", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("key_dtype", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("q_pos0", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_st", ctypes.c_int64),
                ("q_sh", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("k_sb", ctypes.c_int64), ("k_st", ctypes.c_int64),
                ("k_scale", ctypes.c_void_p), ("ks_sb", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("w_sb", ctypes.c_int64), ("w_st", ctypes.c_int64),
                ("q_scale", ctypes.c_void_p), ("qs_sb", ctypes.c_int64), ("qs_st", ctypes.c_int64)]


class Attn(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T_q", ctypes.c_int32), ("T_kv", ctypes.c_int32),
                ("H_q", ctypes.c_int32), ("D_qk", ctypes.c_int32), ("D_v", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("q_pos0", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_st", ctypes.c_int64),
                ("q_sh", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("k_sb", ctypes.c_int64), ("k_st", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_sb", ctypes.c_int64), ("v_st", ctypes.c_int64),
                ("out", ctypes.c_void_p), ("o_sb", ctypes.c_int64), ("o_st", ctypes.c_int64),
                ("o_sh", ctypes.c_int64)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m long_context_sparse_idx_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)
    lib.idx_score_topk.argtypes = [ctypes.POINTER(Indexer), p, i64, i64, p, sz, ctypes.c_uint, p]
    lib.idx_score_topk.restype = i32
    lib.sparse_attn.argtypes = [ctypes.POINTER(Attn), p, i64, i64, p, sz, p]
    lib.sparse_attn.restype = i32
    lib.sparse_attn_noalloc.argtypes = [ctypes.POINTER(Attn), p, i64, i64, p]
    lib.sparse_attn_noalloc.restype = i32
    lib.run_layer_group.argtypes = [i32, p, ctypes.POINTER(Indexer), i32, ctypes.POINTER(Attn), p, i32,
                                    i64, i64, i64, p, sz, p, p]
    lib.run_layer_group.restype = i32
    lib.idx_overlap.argtypes = [p, i64, i64, p, i64, i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, p, p]
    lib.idx_overlap.restype = i32
    lib.lcsi_score_ld.argtypes = [ctypes.c_int32]
    lib.lcsi_score_ld.restype = i64
    lib.lcsi_strerror.argtypes = [i32]
    lib.lcsi_strerror.restype = ctypes.c_char_p
    return lib


lib = _load()


def strerror(code: int) -> str:
    return lib.lcsi_strerror(code).decode()


def score_ld(T_kv: int) -> int:
    return int(lib.lcsi_score_ld(T_kv))


def _check(rc: int, where: str):
    if rc != 0:
        raise LcsiError(rc, where)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)


# ------------------------------------------------------------- descriptors

_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _inner(t: torch.Tensor, name: str, dims: int, dtypes):
    """The library takes strides for the outer dimensions only: the last
    one must be contiguous."""
    _need(t.dim() == dims, f"{name}: expected {dims} dimensions, got {tuple(t.shape)}")
    _need(t.dtype in dtypes, f"{name}: dtype {t.dtype} not in {dtypes}")
    _need(t.shape[-1] <= 1 or t.stride(-1) == 1, f"{name}: the last dimension must be contiguous")


def indexer_desc(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, top_k: int, q_pos0: int,
                 k_scale: Optional[torch.Tensor] = None, T_kv: Optional[int] = None,
                 q_scale: Optional[torch.Tensor] = None) -> Indexer:
    """q [B,T_q,H,D] bf16, or fp8 e4m3 bytes (uint8 / float8_e4m3fn) with
    q_scale [B,T_q,H] fp32; k [B,T_kv,D] bf16 or fp8 e4m3 bytes with k_scale
    [B,T_kv] fp32; w [B,T_q,H] fp32.  T_kv (default k.shape[1]) may name a
    prefix of the keys, never more than k holds."""
    _inner(q, "q", 4, (torch.bfloat16,) + _FP8)
    _inner(k, "k", 3, (torch.bfloat16,) + _FP8)
    _inner(w, "w", 3, (torch.float32,))
    B, T_q, H, D = q.shape
    fp8 = k.dtype in _FP8
    q8 = q.dtype in _FP8
    _need(tuple(k.shape[::2]) == (B, D) and tuple(w.shape) == (B, T_q, H), "q, k, w: shapes do not agree")
    n_kv = k.shape[1] if T_kv is None else int(T_kv)
    _need(0 < n_kv <= k.shape[1], f"T_kv={n_kv} outside 1..{k.shape[1]} (the keys k holds)")
    if fp8:
        _need(k_scale is not None, "k_scale is required with fp8 keys")
        _inner(k_scale, "k_scale", 2, (torch.float32,))
        _need(k_scale.shape[0] == B and k_scale.shape[1] >= n_kv, "k_scale: expected [B, >=T_kv]")
    if q8:
        _need(q_scale is not None, "q_scale is required with fp8 queries")
        _inner(q_scale, "q_scale", 3, (torch.float32,))
        _need(tuple(q_scale.shape) == (B, T_q, H), "q_scale: expected [B, T_q, H]")
    d = Indexer()
    d.B, d.T_q, d.H_I, d.D_I, d.top_k = B, T_q, H, D, top_k
    d.T_kv = n_kv
    d.key_dtype = LCSI_KEY_FP8_E4M3 if fp8 else LCSI_KEY_BF16
    d.q_dtype = LCSI_Q_FP8_E4M3 if q8 else LCSI_Q_BF16
    d.q_pos0 = q_pos0
    d.q, (d.q_sb, d.q_st, d.q_sh) = q.data_ptr(), q.stride()[:3]
    d.k, (d.k_sb, d.k_st) = k.data_ptr(), k.stride()[:2]
    if fp8:
        d.k_scale, d.ks_sb = k_scale.data_ptr(), k_scale.stride(0)
    if q8:
        d.q_scale, (d.qs_sb, d.qs_st) = q_scale.data_ptr(), q_scale.stride()[:2]
    d.w, (d.w_sb, d.w_st) = w.data_ptr(), w.stride()[:2]
    return d


def preset_desc(B: int, T_q: int, T_kv: int, q_pos0: int, top_k: int) -> Indexer:
    d = Indexer()
    d.B, d.T_q, d.T_kv, d.q_pos0, d.top_k = B, T_q, T_kv, q_pos0, top_k
    return d


def attn_desc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, top_k: int,
              q_pos0: int, sm_scale: float, T_kv: Optional[int] = None) -> Attn:
    """q [B,T_q,H,Dqk]; k [B,T_kv,Dqk]; v [B,T_kv,Dv] (may be a column view of
    k); out [B,T_q,H,Dv]; all bf16.  T_kv (default k.shape[1]) may name a
    prefix of the keys, never more than k and v hold."""
    for t, name, dims in ((q, "q", 4), (k, "k", 3), (v, "v", 3), (out, "out", 4)):
        _inner(t, name, dims, (torch.bfloat16,))
    B, T_q, H, Dqk = q.shape
    Dv = v.shape[-1]
    _need(k.shape[0] == B and k.shape[2] == Dqk, f"k: expected [{B}, T_kv, {Dqk}], got {tuple(k.shape)}")
    _need(v.shape[0] == B and v.shape[1] == k.shape[1],
          f"v: expected [{B}, {k.shape[1]}, Dv] like k, got {tuple(v.shape)}")
    _need(tuple(out.shape) == (B, T_q, H, Dv), f"out: expected {(B, T_q, H, Dv)}, got {tuple(out.shape)}")
    n_kv = k.shape[1] if T_kv is None else int(T_kv)
    _need(0 < n_kv <= k.shape[1], f"T_kv={n_kv} outside 1..{k.shape[1]} (the rows k and v hold)")
    d = Attn()
    d.B, d.T_q, d.H_q, d.D_qk, d.D_v, d.top_k = B, T_q, H, Dqk, Dv, top_k
    d.T_kv = n_kv
    d.sm_scale = sm_scale
    d.q_pos0 = q_pos0
    d.q, (d.q_sb, d.q_st, d.q_sh) = q.data_ptr(), q.stride()[:3]
    d.k, (d.k_sb, d.k_st) = k.data_ptr(), k.stride()[:2]
    d.v, (d.v_sb, d.v_st) = v.data_ptr(), v.stride()[:2]
    d.out, (d.o_sb, d.o_st, d.o_sh) = out.data_ptr(), out.stride()[:3]
    return d


def _check_idx(idx: torch.Tensor, desc, name: str = "idx"):
    """An index tensor for rows (B, T_q) of `desc`: [B, T_q, >= top_k] int32,
    innermost dimension contiguous."""
    _inner(idx, name, 3, (torch.int32,))
    _need(tuple(idx.shape[:2]) == (desc.B, desc.T_q) and idx.shape[2] >= desc.top_k,
          f"{name}: expected [{desc.B}, {desc.T_q}, >={desc.top_k}], got {tuple(idx.shape)}")


def _elements_from(t: torch.Tensor) -> int:
    """int32 elements addressable from t's first element to the end of its storage."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


# -------------------------------------------------------------------- calls

def idx_score_topk_ws_bytes(desc: Indexer, flags: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.idx_score_topk(ctypes.byref(desc), None, 0, 0, None, ctypes.byref(n), flags, None),
           "idx_score_topk(query)")
    return n.value


def idx_score_topk(desc: Indexer, idx: Optional[torch.Tensor], ws: torch.Tensor, flags: int = 0,
                   stream=None):
    """Run the indexer of one F layer; idx [B,T_q,>=top_k] int32 (or a view of
    an index-cache slot), ws: score workspace (see idx_score_topk_ws_bytes)."""
    cap = ctypes.c_size_t(ws.numel() * ws.element_size())
    if idx is not None:
        _check_idx(idx, desc)
        sb, st = idx.stride()[:2]
    else:
        _need(flags & LCSI_SCORES_ONLY, "idx is required unless flags has LCSI_SCORES_ONLY")
        sb = st = 0
    _check(lib.idx_score_topk(ctypes.byref(desc), _ptr(idx), sb, st, _ptr(ws), ctypes.byref(cap),
                              flags, _stream(stream)), "idx_score_topk")


def sparse_attn_ws_bytes(desc: Attn) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.sparse_attn(ctypes.byref(desc), None, 0, 0, None, ctypes.byref(n), None),
           "sparse_attn(query)")
    return n.value


def sparse_attn(desc: Attn, idx: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None):
    """Sparse attention of one layer over idx [B,T_q,>=top_k] int32."""
    _check_idx(idx, desc)
    sb, st = idx.stride()[:2]
    if ws is None:
        need = sparse_attn_ws_bytes(desc)
        ws = _ws(need, idx.device)
    cap = ctypes.c_size_t(ws.numel() * ws.element_size()) if ws is not None else None
    _check(lib.sparse_attn(ctypes.byref(desc), _ptr(idx), sb, st, _ptr(ws),
                           ctypes.byref(cap) if cap is not None else None, _stream(stream)),
           "sparse_attn")


def sparse_attn_noalloc(desc: Attn, idx: torch.Tensor, stream=None):
    """sparse_attn with the library's static device scratch instead of a
    workspace (nothing is allocated, here or in the library)."""
    _check_idx(idx, desc)
    sb, st = idx.stride()[:2]
    _check(lib.sparse_attn_noalloc(ctypes.byref(desc), _ptr(idx), sb, st, _stream(stream)),
           "sparse_attn_noalloc")


def run_layer_group(pattern: Sequence[int], idx_descs: Sequence[Indexer], attn_descs: Sequence[Attn],
                    idx_cache: torch.Tensor, n_slots: int, slot_stride: int, idx_sb: int, idx_st: int,
                    ws: Optional[torch.Tensor] = None, events=None, stream=None):
    """The F/S loop.  idx_cache: int32 device buffer holding n_slots slots
    (slot s at element s*slot_stride, row (b, t) at b*idx_sb + t*idx_st)."""
    L = len(pattern)
    _need(idx_cache.dtype == torch.int32, "idx_cache: expected int32")
    if attn_descs:
        a0 = attn_descs[0]
        last = (n_slots - 1) * slot_stride + (a0.B - 1) * idx_sb + (a0.T_q - 1) * idx_st + a0.top_k
        _need(min(slot_stride, idx_sb, idx_st) >= 0 and last <= _elements_from(idx_cache),
              f"idx_cache: {n_slots} slots of [{a0.B}, {a0.T_q}, {a0.top_k}] with strides "
              f"({slot_stride}, {idx_sb}, {idx_st}) reach past its storage")
    pat = (ctypes.c_uint8 * L)(*[1 if x else 0 for x in pattern])
    nf = len(idx_descs)
    ia = (Indexer * max(nf, 1))(*idx_descs)
    aa = (Attn * L)(*attn_descs)
    if ws is None:
        need = layer_group_ws_bytes(pattern, idx_descs, attn_descs, idx_cache, n_slots, slot_stride,
                                    idx_sb, idx_st)
        ws = _ws(need, idx_cache.device)
    cap = ctypes.c_size_t(ws.numel() * ws.element_size()) if ws is not None else None
    ev = None
    if events is not None:
        # torch creates its events lazily on the first record; create them
        # here so the library receives live hipEvent_t handles.
        for e in events:
            if e is not None and not e.cuda_event:
                e.record(torch.cuda.current_stream() if stream is None else stream)
        ev = (ctypes.c_void_p * (4 * L))(*[e.cuda_event if e is not None else 0 for e in events])
    _check(lib.run_layer_group(L, pat, ia, nf, aa, _ptr(idx_cache), n_slots, slot_stride, idx_sb, idx_st,
                               _ptr(ws), ctypes.byref(cap) if cap is not None else None, ev,
                               _stream(stream)), "run_layer_group")
    return ws


def layer_group_ws_bytes(pattern, idx_descs, attn_descs, idx_cache, n_slots, slot_stride, idx_sb,
                         idx_st) -> int:
    L = len(pattern)
    pat = (ctypes.c_uint8 * L)(*[1 if x else 0 for x in pattern])
    nf = len(idx_descs)
    ia = (Indexer * max(nf, 1))(*idx_descs)
    aa = (Attn * L)(*attn_descs)
    n = ctypes.c_size_t(0)
    _check(lib.run_layer_group(L, pat, ia, nf, aa, _ptr(idx_cache), n_slots, slot_stride, idx_sb, idx_st,
                               None, ctypes.byref(n), None, None), "run_layer_group(query)")
    return n.value


def idx_overlap(a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    """Per-row count of positions present in both index lists a, b
    [B, T_q, k] int32 (ascending, -1 padded); returns int32 [B, T_q]."""
    _inner(a, "a", 3, (torch.int32,))
    _inner(b, "b", 3, (torch.int32,))
    _need(b.shape == a.shape, f"a, b: shapes {tuple(a.shape)} and {tuple(b.shape)} differ")
    B, T_q, k = a.shape
    counts = torch.empty((B, T_q), dtype=torch.int32, device=a.device)
    _check(lib.idx_overlap(_ptr(a), a.stride(0), a.stride(1), _ptr(b), b.stride(0), b.stride(1),
                           B, T_q, k, _ptr(counts), _stream(stream)), "idx_overlap")
    return counts
