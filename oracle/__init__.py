"""CPU oracle for the sparse-index hot path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It is the plain, slow, obviously correct
reference the GPU library is checked against; it shares no code with the GPU
path and never imports it.

What it computes (the pages describe the method in prose; see the C file for
the arithmetic):

* ``score_select`` -- the indexer score of each query row against its causal
  keys, ``score[t,s] = sum_h w[t,h]*max(0, q[t,h,:].k[s,:])`` for ``s <= p_t``,
  rounded once to fp32, and the top-k positions of that row (ties to the
  lower position, ascending, padded with -1).  IndexCache news article
  (app.myzaker.com), section "IndexCache"; IndexShare term page
  (earlyterms.com), opening definition ("dot product + top-k").
* ``select`` -- the top-k step alone, on given fp32 score rows.
* ``attn`` -- softmax attention of every query head over only the selected
  rows, in double, rounded once to bf16.  IndexShare explainer (yun88.com),
  section on the hidden indexer cost (attention over the top-k only).
* ``layer_group`` -- the F/S loop: an F layer computes and caches its index
  set, an S layer reuses the most recent F layer's set and still runs its own
  attention.  IndexCache article (linkstar.cloud), section on adjacent layers
  repeating work (F and S layers); IndexShare explainer (yun88.com), section
  on the sharing mechanism (S layers keep their own attention weights).

Every function is pinned by ``tests/test_oracle_pins.py`` against brute force,
closed forms and hand-derived fixtures; nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lcsi_oracle.c")
# LCSI_ORACLE_LIB names another build of the same source to load instead
# (the mutation test points it at deliberately broken copies); it is never
# rebuilt here.
_LIB_OVERRIDE = os.environ.get("LCSI_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None


GCC_FLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE", "-Wall"]


def compile_source(src: str, out: str) -> None:
    """gcc the C oracle source `src` into the shared library `out`."""
    subprocess.run(["gcc", *GCC_FLAGS, "-o", out, src, "-lm", "-lpthread"], check=True)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    lib = os.path.join(_HERE, "liboracle.so")
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp"
        compile_source(_SRC, tmp)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_fp8e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8e4m3_to_double.restype = ctypes.c_double
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_score_select_rows.argtypes = [
            i32, p, p, p, i32, p, p, p, i32, i64, i32, i32, i32, p, i64, p, i32]
        lib.oracle_score_select_rows.restype = i32
        lib.oracle_select_rows.argtypes = [i32, p, i64, p, i32, p, i32]
        lib.oracle_select_rows.restype = i32
        lib.oracle_attn_rows.argtypes = [
            i32, p, p, i64, p, i64, p, i32, i32, i32, i32, ctypes.c_double, p, i32]
        lib.oracle_attn_rows.restype = i32
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- decoding

def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits) & 0xFFFF)


def fp8e4m3_to_double(byte: int) -> float:
    return _load().oracle_fp8e4m3_to_double(int(byte) & 0xFF)


def double_to_bf16(x: float) -> int:
    return int(_load().oracle_double_to_bf16(float(x)))


# ------------------------------------------------------------ score / select

def score_select(q_rows, w_rows, keys, pos, top_k, k_scale=None,
                 want_scores=True, threads=None, q_scale=None):
    """Indexer score + top-k for a list of query rows sharing one key array.

    q_rows : uint16 [R, H, D] (bf16 bit patterns) or uint8 [R, H, D] (fp8
             e4m3 bytes, then q_scale float32 [R, H] gives each head's scale)
    w_rows : float32 [R, H]
    keys   : uint16 [N, D] (bf16 bits) or uint8 [N, D] (fp8 e4m3 bytes)
    pos    : int64 [R] absolute position p of each row (it sees keys 0..p)
    k_scale: float32 [N] per-key scale for fp8 keys, else None
    Returns (scores float32 [R, max_p+1] or None, idx int32 [R, top_k]).
    Entries of a score row past its p are left at 0.
    """
    q_fp8 = np.asarray(q_rows).dtype == np.uint8
    q_rows = _c(q_rows, np.uint8 if q_fp8 else np.uint16)
    qs = _c(q_scale, np.float32) if q_fp8 else None
    w_rows = _c(w_rows, np.float32)
    pos = _c(pos, np.int64)
    R, H, D = q_rows.shape
    assert not q_fp8 or qs.shape == (R, H)
    key_fp8 = keys.dtype == np.uint8
    keys = _c(keys, np.uint8 if key_fp8 else np.uint16)
    assert keys.shape[1] == D and keys.shape[0] > int(pos.max(initial=-1))
    ks = _c(k_scale, np.float32) if key_fp8 else None
    n_max = int(pos.max(initial=-1)) + 1
    scores = np.zeros((R, max(n_max, 1)), np.float32) if want_scores else None
    idx = np.empty((R, top_k), np.int32)
    _load().oracle_score_select_rows(
        R, _ptr(pos), _ptr(q_rows), _ptr(qs), int(q_fp8), _ptr(w_rows), _ptr(keys), _ptr(ks),
        int(key_fp8), D, H, D, top_k, _ptr(scores),
        scores.shape[1] if want_scores else 0, _ptr(idx),
        threads or default_threads())
    return scores, idx


def select(scores, n, top_k, threads=None):
    """Top-k on given fp32 score rows; row r considers entries [0, n[r])."""
    scores = _c(scores, np.float32)
    R = scores.shape[0]
    n = _c(np.broadcast_to(np.asarray(n, np.int64), (R,)), np.int64)
    idx = np.empty((R, top_k), np.int32)
    _load().oracle_select_rows(R, _ptr(scores), scores.shape[1], _ptr(n), top_k,
                               _ptr(idx), threads or default_threads())
    return idx


# ---------------------------------------------------------------- attention

def attn(q_rows, K, V, idx, tau, threads=None):
    """Sparse attention for rows sharing one K/V array.

    q_rows : uint16 [R, H, Dqk] (bf16 bits); K : uint16 [N, Dqk-or-wider]
    (row stride = K.shape[1], the first Dqk columns used); V : uint16
    [N, >= Dv] likewise; idx : int32 [R, top_k].  Returns uint16 [R, H, Dv]
    (bf16 bits).  ``V`` may be a column slice of the K array (MLA-style
    shared row): pass the full rows and ``Dv`` through ``V.shape``.
    """
    q_rows = _c(q_rows, np.uint16)
    R, H, Dqk = q_rows.shape
    idx = _c(idx, np.int32)
    top_k = idx.shape[1]
    Kc = np.ascontiguousarray(K)
    k_ld = Kc.shape[1]
    if isinstance(V, tuple):  # (array, Dv): V is the first Dv columns of array
        Vc, Dv = np.ascontiguousarray(V[0]), V[1]
    else:
        Vc = np.ascontiguousarray(V)
        Dv = Vc.shape[1]
    v_ld = Vc.shape[1]
    assert Kc.dtype == np.uint16 and Vc.dtype == np.uint16
    out = np.empty((R, H, Dv), np.uint16)
    _load().oracle_attn_rows(R, _ptr(q_rows), _ptr(Kc), k_ld, _ptr(Vc), v_ld,
                             _ptr(idx), top_k, H, Dqk, Dv, float(tau),
                             _ptr(out), threads or default_threads())
    return out


# -------------------------------------------------------------- layer group

def layer_group(pattern, f_layers, attn_layers, pos, top_k, threads=None):
    """The F/S layer loop on a list of query rows.

    pattern     : sequence of 1 (F) / 0 (S), one per layer; must start with F.
    f_layers    : one dict per F layer, in order, with keys q (uint16 [R,H,D]),
                  w (float32 [R,H]), keys (uint16/uint8 [N,D]), k_scale.
    attn_layers : one dict per layer with q (uint16 [R,Hq,Dqk]), K, V, tau.
    Returns (list of per-layer idx arrays, list of per-layer outputs).
    An S layer uses the index array of the most recent F layer (the nearest
    preceding F) and its own attention inputs.
    """
    idx_per_layer, outs = [], []
    cur = None
    fi = 0
    for l, is_f in enumerate(pattern):
        if is_f:
            a = f_layers[fi]
            fi += 1
            _, cur = score_select(a["q"], a["w"], a["keys"], pos, top_k,
                                  k_scale=a.get("k_scale"), want_scores=False,
                                  threads=threads)
        elif cur is None:
            raise ValueError("pattern starts with an S layer: no F layer to reuse")
        b = attn_layers[l]
        outs.append(attn(b["q"], b["K"], b["V"], cur, b["tau"], threads=threads))
        idx_per_layer.append(cur)
    if fi != len(f_layers):
        raise ValueError("number of F layers does not match the indexer inputs")
    return idx_per_layer, outs


# ------------------------------------------------------------------ overlap

def overlap_counts(a, b):
    """Per row, the number of positions (entries >= 0) present in both index
    lists: a, b int32 [R, k] -> int64 [R].  Plain set intersection."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape
    return np.array([np.intersect1d(a[r][a[r] >= 0], b[r][b[r] >= 0]).size for r in range(a.shape[0])],
                    np.int64)
