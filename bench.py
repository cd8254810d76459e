"""Benchmark of the sparse-index hot path on one MI355X.

A step is one pass of the whole path over the 200K-token prefill workload:
25 chunks of up to 8192 query rows against the resident keys, each chunk
through run_layer_group with 4 layers F,S,S,S (indexer score + top-k in the F
layer, index-cache reuse, sparse attention in every layer).

Headline metric: indexer + top-k prefill query-tok/s at 200K context =
200000 / (indexer time per step), where the indexer time is the sum over
chunks of the F layer's score + select kernels, timed with HIP events that
run_layer_group records on the launch stream.  The JSON line also carries the
whole-path rate, the FSSS vs all-F speedup (one all-F pass after the timed
steps), the score kernel's MFMA roofline (and its fraction of the measured
matrix-core ceiling), the HBM traffic of the score, select and attention
kernels from the committed counter runs, and the CPU oracle's rate on a
bounded sample of rows.  After the headline the decode workloads at 131K and
1M context and the 1M prefill chunk are timed against their all-F patterns
(steps timed back to back without per-layer events; one more step with
events gives the per-kernel split).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                    [--no-allf] [--no-ceilings] [--no-secondary]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_sparse_idx_amd import inputs, lcsi  # noqa: E402
from long_context_sparse_idx_amd.runner import Workload, pairs_in_chunk  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

SECONDARY = ("decode131k", "decode1m", "prefill1m")
COUNTERS_JSON = os.path.join(ROOT, "profiles", "hbm_counters.json")
CSRC = os.path.join(ROOT, "long_context_sparse_idx_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_entries(workload: str, kernel_prefix: str):
    """Every committed FETCH_SIZE / WRITE_SIZE entry of this workload whose
    kernel name starts with kernel_prefix (all template variants), or None
    when there is none or a source one was taken from has changed since."""
    try:
        with open(COUNTERS_JSON) as f:
            doc = json.load(f)
    except OSError:
        return None
    es = [e for e in doc.get("entries", [])
          if e["workload"] == workload and e["kernel"].startswith(kernel_prefix)]
    if not es or not all(source_sha(s) == h for e in es for s, h in e["sources"].items()):
        return None
    return es


def hbm_stage_for(workload: str, primary: str, others, stage_ms: float):
    """A stage of the path (score, selection, attention with its merges): its
    HBM bytes per call = the counted bytes of every kernel of the stage (all
    template variants of each name) over the calls in the counted run (one
    launch of a `primary` kernel per call), against the stage's time per call
    measured in this run; None without a current counter entry."""
    ps = counter_entries(workload, primary)
    if ps is None or stage_ms <= 0:
        return None
    parts = ps + [e for o in others for e in (counter_entries(workload, o) or [])]
    total = sum(e["bytes_per_launch"] * e["dispatches"] for e in parts) / sum(e["dispatches"] for e in ps)
    gbs = total / (stage_ms / 1e3) / 1e9
    return {"kernels": [e["kernel"] for e in parts], "bytes_per_call": int(total),
            "call_ms_this_run": round(stage_ms, 4), "GBps": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def counter_entry(workload: str, kernel_prefix: str, kernel_suffix: str = ""):
    """The committed FETCH_SIZE / WRITE_SIZE entry of a kernel (HBM bytes per
    launch), or None when there is none for this workload or a source it was
    taken from has changed since."""
    try:
        with open(COUNTERS_JSON) as f:
            doc = json.load(f)
    except OSError:
        return None
    for e in doc.get("entries", []):
        if (e["workload"] != workload or not e["kernel"].startswith(kernel_prefix)
                or not e["kernel"].endswith(kernel_suffix)):
            continue
        if all(source_sha(s) == h for s, h in e["sources"].items()):
            return e
    return None


def cpu_baseline(path: Workload, max_rows: int | None = None):
    """The oracle's indexer + top-k on a bounded sample of rows: evenly
    spaced query rows of sequence 0 for a prefill workload, the new token of
    the first few sequences for decode."""
    import oracle
    wl = path.wl
    threads = oracle.default_threads()
    x = path.idx_in[path.pattern_f[0]]

    def seq_arrays(b):
        if wl.key_fp8:
            return x["k"][b].cpu().numpy(), x["k_scale"][b].cpu().numpy()
        return x["k"][b].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), None

    def rows_of(b, rows):
        r = torch.as_tensor(rows, device=x["q"].device)
        if wl.q_fp8:
            q = x["q"][b].index_select(0, r).cpu().numpy()
            qs = x["q_scale"][b].index_select(0, r).cpu().numpy()
        else:
            q = x["q"][b].index_select(0, r).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            qs = None
        return q, x["w"][b].index_select(0, r).cpu().numpy(), qs

    t0 = time.time()
    if wl.n_q > 1:
        R = max_rows or max(8, 4 * threads)
        pos = np.array([wl.q_pos0 + int((i + 0.5) * wl.n_q / R) for i in range(R)], np.int64)
        q, w, qs = rows_of(0, pos - wl.q_pos0)
        keys, ks = seq_arrays(0)
        t0 = time.time()
        oracle.score_select(q, w, keys, pos, wl.top_k, k_scale=ks, want_scores=False, threads=threads,
                            q_scale=qs)
        what = f"{R} evenly spaced rows of sequence 0 (positions {pos[0]}..{pos[-1]})"
    else:
        R = max_rows or min(wl.B, 4)
        dt = 0.0
        for b in range(R):
            q, w, qs = rows_of(b, [0])
            keys, ks = seq_arrays(b)
            t1 = time.time()
            oracle.score_select(q, w, keys, np.array([wl.q_pos0], np.int64), wl.top_k, k_scale=ks,
                                want_scores=False, threads=threads, q_scale=qs)
            dt += time.time() - t1
        t0 = time.time() - dt
        what = f"the new token of sequences 0..{R - 1} (position {wl.q_pos0}), one row per call"
        threads = 1     # the oracle spreads rows over threads; one row runs on one
    dt = time.time() - t0
    return {"value": R / dt, "unit": "query-tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of the {wl.name} workload, indexer score + top-k, "
                      f"{dt:.1f} s wall on {threads} threads"}


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def mfma_ceiling():
    """The score kernel's matrix-core instruction stream with nothing else
    (libceiling.so): B operands from registers (mode 0) and from LDS with the
    score kernel's reads (mode 1), on N(0,1)/8 bf16 operands.  TFLOP/s."""
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_idx_amd", "libceiling.so"))
    lib.lcsi_ceiling_data_elems.restype = ctypes.c_size_t
    lib.lcsi_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.lcsi_ceiling_mfma.restype = ctypes.c_int
    n = lib.lcsi_ceiling_data_elems()
    g = torch.Generator(device="cuda").manual_seed(5)
    data = (torch.randn(n, device="cuda", generator=g) / 8).to(torch.bfloat16)
    n_wg, blocks = 2048, 1024
    out = torch.empty(n_wg * 8, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for mode in (0, 1):
        def launch():
            rc = lib.lcsi_ceiling_mfma(ctypes.c_void_p(data.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                       n_wg, blocks, mode, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"lcsi_ceiling_mfma: {rc}")
        for _ in range(2):
            launch()
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        flops = n_wg * 8 * blocks * 16 * 32768.0 * reps
        res[("mfma_only_regs" if mode == 0 else "mfma_lds_reads") + "_TFLOPs"] = round(
            flops / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    del data, out
    return res


def measured_ceilings():
    """Practical ceilings on this GPU, for context beside the datasheet peaks:
    a library bf16 GEMM (8192^3, entries N(0,1)/8 like the indexer inputs),
    the score kernel's MFMA stream alone (libceiling.so), a 4 GiB
    device-to-device copy, a 4 GiB read-only reduction (torch), a 4 GiB
    plain streaming read and a gather of one decode attention layer's rows
    (libceiling.so).  All run after the timed region."""
    g = torch.Generator(device="cuda").manual_seed(0)
    n = 8192
    a = (torch.randn(n, n, device="cuda", generator=g) / 8).to(torch.bfloat16)
    b = (torch.randn(n, n, device="cuda", generator=g) / 8).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2 * n ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b
    res = {"bf16_gemm_8192_TFLOPs": round(gemm, 1), "bf16_gemm_frac_of_peak": round(gemm / PEAK_BF16_TFLOPS, 4)}
    res.update(mfma_ceiling())
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * src.numel() * 4 * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del dst
    s = src.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        s = src.sum()
    e1.record()
    torch.cuda.synchronize()
    read = src.numel() * 4 * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    stream_read = read_ceiling(src)
    del src, s
    torch.cuda.empty_cache()
    res.update({"copy_4GiB_GBps": round(copy, 1), "copy_frac_of_peak": round(copy / PEAK_HBM_GBS, 4),
                "read_4GiB_sum_GBps": round(read, 1), "read_frac_of_peak": round(read / PEAK_HBM_GBS, 4),
                "read_4GiB_stream_GBps": round(stream_read, 1),
                "read_stream_frac_of_peak": round(stream_read / PEAK_HBM_GBS, 4)})
    res.update(gather_ceiling())
    return res


def read_ceiling(buf: torch.Tensor) -> float:
    """A plain streaming read of `buf` (libceiling.so): GB/s."""
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_idx_amd", "libceiling.so"))
    lib.lcsi_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.lcsi_ceiling_read.restype = ctypes.c_int
    n_wg = 4096
    out = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    nbytes = buf.numel() * buf.element_size()

    def launch():
        rc = lib.lcsi_ceiling_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nbytes),
                                   ctypes.c_void_p(out.data_ptr()), n_wg, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"lcsi_ceiling_read: {rc}")
    launch()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9


def gather_ceiling() -> dict:
    """The sparse attention's memory pattern without its arithmetic
    (libceiling.so): the rows of one decode131k attention layer -- 32
    sequences x 2048 distinct random rows of 1152 bytes out of 131073 each,
    every row gathered once -- copied into LDS by 512 workgroups (two per
    CU) of four 32-row lists, one list in flight while the last is read back."""
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_idx_amd", "libceiling.so"))
    lib.lcsi_ceiling_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lcsi_ceiling_gather.restype = ctypes.c_int
    B, N, k, rowb = 32, 131073, 2048, 1152
    kv = torch.empty(B * N * rowb // 4, dtype=torch.int32, device="cuda")  # contents do not matter
    g = torch.Generator(device="cuda").manual_seed(1)
    rows = torch.stack([torch.randperm(N, generator=g, device="cuda")[:k].sort().values + b * N
                        for b in range(B)]).to(torch.int32).contiguous()   # [B, k] global row numbers
    n_wg, tiles = B * k // 128, 4
    out = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.lcsi_ceiling_gather(ctypes.c_void_p(kv.data_ptr()), B * N, rowb, ctypes.c_void_p(rows.data_ptr()),
                                     n_wg, tiles, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"lcsi_ceiling_gather: {rc}")
    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del kv, rows, out
    torch.cuda.empty_cache()
    gbs = B * k * rowb / (ms / 1e3) / 1e9
    return {"gather_1152B_rows_decode131k_us": round(ms * 1e3, 2), "gather_1152B_rows_GBps": round(gbs, 1),
            "gather_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def split_ms(events, nchunk, L):
    """Score / select / attention ms of one step from run_layer_group's
    per-layer events."""
    sc = se = at = 0.0
    for c in range(nchunk):
        ev = events[c]
        for l in range(L):
            sc += ev[4 * l].elapsed_time(ev[4 * l + 1])
            se += ev[4 * l + 1].elapsed_time(ev[4 * l + 2])
            at += ev[4 * l + 2].elapsed_time(ev[4 * l + 3])
    return sc, se, at


def score_ms_of(events, chunks, L, pattern):
    """Score ms of the given chunks of one step from run_layer_group's
    per-layer events (F layers only)."""
    return sum(events[c][4 * l].elapsed_time(events[c][4 * l + 1]) for c in chunks for l in range(L) if pattern[l])


def time_steps(path, plan, steps, warmup):
    """ms per step over `steps` back-to-back steps (no per-layer events), and
    one more step with per-layer events: (ms/step, score ms, select ms,
    attention ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        path.step(plan)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record(stream)
    for _ in range(steps):
        path.step(plan)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    L = len(plan[0])
    nchunk = len(plan[1])
    ev = [_events(4 * L) for _ in range(nchunk)]
    path.step(plan, ev)
    torch.cuda.synchronize()
    sc, se, at = split_ms(ev, nchunk, L)
    return ms, sc, se, at


def decode_graph(path, plan, steps):
    """A decode step as one HIP graph replay against eager launches: steps
    back to back (throughput), and one token at a time with the host waiting
    for each step (the latency a decode loop that samples between tokens
    sees, where the host's launch rate can fall behind short kernels)."""
    B = path.wl.B
    g = path.capture(plan)
    g.replay()
    torch.cuda.synchronize()

    def per_token(fn):
        ts = []
        for _ in range(steps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(ts))

    e0, e1 = _events(2)
    e0.record(torch.cuda.current_stream())
    for _ in range(steps):
        g.replay()
    e1.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / steps
    lat_eager = per_token(lambda: path.step(plan))
    lat_graph = per_token(g.replay)
    del g
    return {"graph_ms_per_step": round(ms_graph, 4), "graph_tok/s": round(B / (ms_graph / 1e3), 1),
            "token_latency_ms_eager": round(lat_eager, 4), "token_latency_ms_graph": round(lat_graph, 4),
            "token_latency_note": "host clock around one step plus a synchronize, median of the timed steps"}


def secondary(name: str, steps: int, warmup: int):
    """One of the other workloads, its layer pattern against all-F."""
    wl = inputs.WORKLOADS[name]
    L = wl.n_layers
    t0 = time.time()
    path = Workload(wl, f_layers=range(L), log=log)
    pat = path.plan(wl.pattern)
    ms, sc, se, at = time_steps(path, pat, steps, warmup)
    allf = path.plan(tuple(1 for _ in range(L)))
    ms_f, sc_f, se_f, at_f = time_steps(path, allf, steps, warmup)
    n_tok = wl.B * wl.n_q
    unit = "tok/s" if wl.T_q == 1 else "query-tok/s"
    out = {
        "pattern": "".join("F" if f else "S" for f in wl.pattern),
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4),
        unit: round(n_tok / (ms / 1e3), 1),
        "indexer_" + unit: round(n_tok / ((sc + se) / 1e3), 1),
        "allF_ms_per_step": round(ms_f, 4),
        "speedup_vs_allF": round(ms_f / ms, 3),
        "split_ms_one_evented_step": {"score": round(sc, 4), "select": round(se, 4), "attention": round(at, 4),
                                      "allF_score": round(sc_f, 4), "allF_select": round(se_f, 4),
                                      "allF_attention": round(at_f, 4)},
        "indexer_share_allF": round((sc_f + se_f) / (sc_f + se_f + at_f), 3),
        "indexer_share_pattern": round((sc + se) / (sc + se + at), 3),
    }
    if wl.T_q == 1:
        # decode scores are memory-bound: the key bytes (+ fp8 scales), queries
        # and weights read and the score row written, per F layer, over the
        # evented step's score time
        key_b = wl.D_I * (1 if wl.key_fp8 else 2) + (4 if wl.key_fp8 else 0)
        q_b = wl.D_I * (1 if wl.q_fp8 else 2) + (8 if wl.q_fp8 else 4)
        nbytes = wl.B * (wl.T_kv * (key_b + 4) + wl.H_I * q_b) * sum(wl.pattern)
        out["score_algorithmic_GBps_evented"] = round(nbytes / (sc / 1e3) / 1e9, 1)
        # attention: the gathered KV rows of every layer over the evented
        # step's attention time (the split partials and Q/O not counted)
        kv_b = wl.B * min(wl.top_k, wl.T_kv) * (2 * wl.D_qk) * L
        out["attention_us_per_layer_evented"] = round(at / L * 1e3, 2)
        out["attention_algorithmic_GBps_evented"] = round(kv_b / (at / 1e3) / 1e9, 1)
        # measured HBM traffic per call (committed counter runs of the same
        # sources) over the evented step's time per call
        n_f = sum(wl.pattern)
        out["hbm"] = {
            "source": "bytes per call from profiles/hbm_counters.json; call times from this run's evented step",
            "score": hbm_stage_for(name, "score_splitkey_kernel", (), sc / n_f),
            "select": hbm_stage_for(name, "select_filter_kernel", ("select_final_kernel",), se / n_f),
            "attention": hbm_stage_for(name, "attn_kernel", ("attn_merge_kernel",), at / L),
        }
        try:
            out.update(decode_graph(path, pat, steps))
        except RuntimeError as e:  # a capture failure must not cost the rest of the line
            out["graph_error"] = str(e)[:200]
            torch.cuda.synchronize()
    log(f"[bench] {name}: {ms:.3f} ms/step ({out[unit]:.0f} {unit}), all-F {ms_f:.3f} ms, "
        f"x{out['speedup_vs_allF']} ({time.time() - t0:.1f} s)")
    del path
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill200k", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-allf", action="store_true", help="skip the all-F comparison pass")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the library GEMM / MFMA loop / copy / read ceiling measurements")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the decode 131K, decode 1M and prefill 1M timings after the headline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy and one 1 GiB read-only reduction first "
                         "(references of known size for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no "
              "multi-GPU mode (every step is row-local; a sharded layout is described, not built)",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)          # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        s = src.sum()           # reads 1 GiB, writes a few bytes
        torch.cuda.synchronize()
        del src, dst, s
        log("[bench] calibration: 1 GiB copy and 1 GiB read-only sum done")
    wl = inputs.WORKLOADS[args.workload]
    path = Workload(wl, f_layers=range(wl.n_layers) if not args.no_allf else None, log=log)
    pattern = wl.pattern
    plan = path.plan(pattern)
    plans = plan[1]
    L = wl.n_layers
    nchunk = len(plans)
    events = [_events(4 * L) for _ in range(nchunk)]
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        path.step(plan)
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    # the fused candidate pass (prefill kernel, 16+ heads, a row longer than
    # its candidate slots): the library plans it when its workspace needs
    # the slots; chunks of shorter rows run unfused
    def plan_fused(d):
        return lcsi.idx_score_topk_ws_bytes(d) > lcsi.idx_score_topk_ws_bytes(d, lcsi.LCSI_UNFUSED)
    fused_chunks = [c for c, p in enumerate(plans) if plan_fused(p[3][0])] if wl.T_q > 1 else []

    start, end = _events(2)
    step_ms, idx_ms, score_ms, select_ms, attn_ms, fused_ms = [], [], [], [], [], []
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        path.step(plan, events)
        torch.cuda.synchronize()
        sc, se, at = split_ms(events, nchunk, L)
        fused_ms.append(score_ms_of(events, fused_chunks, L, pattern))
        step_ms.append(s0.elapsed_time(events[-1][-1]))
        score_ms.append(sc)
        select_ms.append(se)
        attn_ms.append(at)
        idx_ms.append(sc + se)
        log(f"[bench] step {i + 1}/{args.steps}: {step_ms[-1]:.1f} ms (score {sc:.1f}, select {se:.1f}, "
            f"attention {at:.1f})")
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    n_q_total = wl.B * wl.n_q
    ms_step = total_ms / args.steps
    idx_mean = float(np.mean(idx_ms))
    value = n_q_total / (idx_mean / 1e3)

    # roofline of the dominant kernel: the indexer score, MFMA-bound for a
    # prefill chunk, HBM-bound for decode (one query row per sequence)
    pairs = sum(pairs_in_chunk(q0, tq) for (q0, tq, _, _, _, _) in plans) * wl.B
    flops_per_pair = 2 * wl.H_I * wl.D_I
    n_f = sum(pattern)
    score_s = float(np.mean(score_ms)) / 1e3
    kdt = "fp8xfp8" if wl.q_fp8 else ("fp8" if wl.key_fp8 else "bf16")

    n_fused = len(fused_chunks)
    fused = n_fused > 0
    peak = PEAK_FP8_TFLOPS if wl.q_fp8 else PEAK_BF16_TFLOPS
    score_launch_ms = float(np.mean(score_ms)) / (nchunk * n_f)
    # (the dominant variant: the fused candidate pass where a chunk plans it)
    score_counters = (counter_entry(wl.name, "score_prefill_kernel", ", true>" if fused else ", false>")
                      if wl.T_q > 1 else counter_entry(wl.name, "score_splitkey_kernel"))
    if wl.T_q > 1:
        # the dominant kernel's own launches: the fused chunks where there are
        # any (their algorithmic flops over their score time: the launch with
        # its zeroing and rescoring launches, ~15 us of a ~10 ms chunk)
        dom = fused_chunks if fused else list(range(nchunk))
        pairs_dom = sum(pairs_in_chunk(plans[c][0], plans[c][1]) for c in dom) * wl.B
        dom_s = (float(np.mean(fused_ms)) if fused else float(np.mean(score_ms))) / 1e3
        achieved = pairs_dom * flops_per_pair * n_f / dom_s / 1e12
        all_achieved = pairs * flops_per_pair * n_f / score_s / 1e12
        score_launch_ms = dom_s * 1e3 / (len(dom) * n_f)
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": score_counters["bytes_per_launch"] if score_counters else None,
                    "kernel": f"score_prefill_kernel<{wl.H_I},{wl.D_I},{kdt}{',fused' if fused else ''}>",
                    "all_chunks": {"achieved": round(all_achieved, 2), "frac": round(all_achieved / peak, 4),
                                   "avg_chunk_ms": round(score_s * 1e3 / (nchunk * n_f), 4),
                                   "note": "every chunk's score phase, the short unfused first chunks included"}}
    else:
        # keys (+ fp8 scale) read once per sequence, queries and weights, score row written
        key_b = wl.D_I * (1 if wl.key_fp8 else 2) + (4 if wl.key_fp8 else 0)
        q_b = wl.D_I * (1 if wl.q_fp8 else 2) + (8 if wl.q_fp8 else 4)
        sc_bytes = wl.B * (wl.T_kv * (key_b + 4) + wl.H_I * q_b) * n_f
        achieved = sc_bytes / score_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": score_counters["bytes_per_launch"] if score_counters else None,
                    "kernel": f"score_splitkey_kernel<{wl.H_I},{wl.D_I},{kdt}>"}
    roofline["launches_per_step"] = (n_fused if fused else nchunk) * n_f
    if fused:
        roofline["unfused_launches_per_step"] = (nchunk - n_fused) * n_f
    roofline["avg_launch_ms"] = round(score_launch_ms, 4)
    # attention: bytes of the gathered KV rows (576 x bf16 per selected index) + Q + O
    sel_per_row = sum(min(wl.top_k, p + 1) for p in range(wl.q_pos0, wl.q_pos0 + wl.n_q)) * wl.B
    attn_bytes = (sel_per_row * wl.D_qk * 2 + n_q_total * wl.H_q * (wl.D_qk + wl.D_v) * 2) * L
    attn_gbs = attn_bytes / (float(np.mean(attn_ms)) / 1e3) / 1e9

    # measured HBM traffic (committed FETCH_SIZE / WRITE_SIZE runs of the
    # same sources) over the launch times measured in this run
    def hbm(entry, launch_ms):
        if entry is None:
            return None
        gbs = entry["bytes_per_launch"] / (launch_ms / 1e3) / 1e9
        return {"kernel": entry["kernel"], "bytes_per_launch": entry["bytes_per_launch"],
                "launch_ms_this_run": round(launch_ms, 4), "GBps": round(gbs, 1),
                "frac": round(gbs / PEAK_HBM_GBS, 4)}

    def hbm_stage(primary, others, stage_ms):
        return hbm_stage_for(wl.name, primary, others, stage_ms)
    select_ms_call = float(np.mean(select_ms)) / (nchunk * n_f)
    hbm_block = {
        "source": "bytes per launch from profiles/hbm_counters.json (rocprofv3 FETCH_SIZE and WRITE_SIZE "
                  "runs of the same kernel sources, scaled by a 1 GiB copy counted in the same runs); "
                  "launch times measured in this run",
        "score": hbm(score_counters, score_launch_ms),
        "select": (hbm_stage("select_kernel", (), select_ms_call) if wl.T_q > 1 else
                   hbm_stage("select_filter_kernel", ("select_final_kernel",), select_ms_call)),
        "attention": hbm_stage("attn_kernel", ("attn_merge_kernel",), float(np.mean(attn_ms)) / (nchunk * L)),
    }

    extra = {}
    if not args.no_allf:
        allf = tuple(1 for _ in range(L))
        plan_f = path.plan(allf)
        path.step(plan_f)
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        ev_f = [_events(4 * L) for _ in range(nchunk)]
        e0.record(stream)
        path.step(plan_f, ev_f)
        e1.record(stream)
        torch.cuda.synchronize()
        allf_ms = e0.elapsed_time(e1)
        idx_f = sum(ev[4 * l].elapsed_time(ev[4 * l + 2]) for ev in ev_f for l in range(L))
        extra["allF_ms_per_step"] = round(allf_ms, 2)
        extra["fsss_speedup_vs_allF"] = round(allf_ms / float(np.mean(step_ms)), 3)
        extra["indexer_share_allF"] = round(idx_f / allf_ms, 3)
        extra["indexer_share_fsss"] = round(idx_mean / float(np.mean(step_ms)), 3)
        log(f"[bench] all-F pass: {allf_ms:.1f} ms")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(path)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} {cpu['unit']} ({cpu['sample']})")
    del path, plan, plans, events
    torch.cuda.empty_cache()

    if not args.no_secondary and wl.name == "prefill200k":
        sec_steps = min(args.steps, 20)
        for name in SECONDARY:
            st, wu = (min(sec_steps, 4), 1) if name == "prefill1m" else (sec_steps, max(args.warmup, 2))
            extra[name] = secondary(name, st, wu)

    if not args.no_ceilings:
        extra["measured_ceilings"] = measured_ceilings()
        if wl.T_q > 1 and not wl.q_fp8:
            ceil = extra["measured_ceilings"]["mfma_lds_reads_TFLOPs"]
            roofline["frac_of_mfma_lds_ceiling"] = round(roofline["achieved"] / ceil, 4)
        # (the gather ceiling is measured on the decode131k layer's shape)
        if "decode131k" in extra:
            extra["decode131k"]["attention_frac_of_gather_ceiling"] = round(
                extra["decode131k"]["attention_algorithmic_GBps_evented"] /
                extra["measured_ceilings"]["gather_1152B_rows_GBps"], 4)
        log(f"[bench] ceilings: {extra['measured_ceilings']}")

    line = {
        "metric": "indexer+top-k prefill query-tok/s at 200K ctx" if wl.name == "prefill200k"
        else f"indexer+top-k query-tok/s ({wl.name})",
        "value": round(value, 1),
        "unit": "query-tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3 (queries and keys)" if wl.q_fp8 else
                  "bf16 (fp8 e4m3 keys widened exactly)" if wl.key_fp8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.q_pos0 + wl.n_q, "B": wl.B, "chunk": wl.T_q,
                   "pattern": "".join("F" if f else "S" for f in pattern), "H_I": wl.H_I,
                   "D_I": wl.D_I, "top_k": wl.top_k, "H_q": wl.H_q, "D_qk": wl.D_qk, "D_v": wl.D_v},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "path_query_tok_s": round(n_q_total / (float(np.mean(step_ms)) / 1e3), 1),
        "ms": {"score": round(float(np.mean(score_ms)), 3), "select": round(float(np.mean(select_ms)), 3),
               "attention": round(float(np.mean(attn_ms)), 3), "indexer": round(idx_mean, 3),
               "step_events": round(float(np.mean(step_ms)), 3)},
        "hbm": hbm_block,
        "attention_algorithmic_GBps": round(attn_gbs, 1),
        "attention_algorithmic_note": "gathered KV rows + Q + O per launch over its time; can exceed the "
                                      "HBM peak where rows repeat within the Infinity Cache (see hbm)",
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
