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
steps), the score kernel's MFMA roofline and the CPU oracle's rate on a
bounded sample of rows.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def score_traffic(wl):
    """HBM bytes per score launch from the committed counter runs, or None
    when the score kernel source changed since they were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "score_traffic.json")) as f:
            t = json.load(f)
        with open(os.path.join(ROOT, "long_context_sparse_idx_amd", "csrc", "score.hip"), "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if t.get("source_sha256") != h or t.get("workload") != wl.name:
        return None
    return t["bytes_per_launch"]


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


def measured_ceilings():
    """Practical ceilings on this GPU, for context beside the datasheet peaks:
    a library bf16 GEMM (8192^3, entries N(0,1)/8 like the indexer inputs) and
    a 4 GiB device-to-device copy.  Both run after the timed region."""
    g = torch.Generator(device="cuda").manual_seed(0)
    n = 8192
    a = (torch.randn(n, n, device="cuda", generator=g) / 8).to(torch.bfloat16)
    b = (torch.randn(n, n, device="cuda", generator=g) / 8).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2 * n ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b
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
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_8192_TFLOPs": round(gemm, 1), "bf16_gemm_frac_of_peak": round(gemm / PEAK_BF16_TFLOPS, 4),
            "copy_4GiB_GBps": round(copy, 1), "copy_frac_of_peak": round(copy / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill200k", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-allf", action="store_true", help="skip the all-F comparison pass")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the library GEMM / device copy ceiling measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first (reference for HBM counters)")
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
        del src, dst
        log("[bench] calibration copy of 1 GiB done")
    wl = inputs.WORKLOADS[args.workload]
    path = Workload(wl, f_layers=range(wl.n_layers) if not args.no_allf else None, log=log)
    pattern = wl.pattern
    plan = path.plan(pattern)
    plans = plan[1]
    L = wl.n_layers
    nchunk = len(plans)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4 * L)] for _ in range(nchunk)]
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        path.step(plan)
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ms, idx_ms, score_ms, select_ms, attn_ms = [], [], [], [], []
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        path.step(plan, events)
        torch.cuda.synchronize()
        sc = se = at = 0.0
        for c in range(nchunk):
            ev = events[c]
            for l in range(L):
                sc += ev[4 * l].elapsed_time(ev[4 * l + 1])
                se += ev[4 * l + 1].elapsed_time(ev[4 * l + 2])
                at += ev[4 * l + 2].elapsed_time(ev[4 * l + 3])
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
    # the fused candidate pass (prefill kernel, 16+ heads, a row longer than
    # its candidate slots): the library plans it when its workspace needs
    # the slots; chunks of shorter rows run unfused
    def plan_fused(d):
        return lcsi.idx_score_topk_ws_bytes(d) > lcsi.idx_score_topk_ws_bytes(d, lcsi.LCSI_UNFUSED)
    n_fused = sum(plan_fused(p[3][0]) for p in plans)
    fused = n_fused > 0
    peak = PEAK_FP8_TFLOPS if wl.q_fp8 else PEAK_BF16_TFLOPS
    if wl.T_q > 1:
        achieved = pairs * flops_per_pair * n_f / score_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": score_traffic(wl),
                    "kernel": f"score_prefill_kernel<{wl.H_I},{wl.D_I},{kdt}{',fused' if fused else ''}>"}
    else:
        # keys (+ fp8 scale) read once per sequence, queries and weights, score row written
        key_b = wl.D_I * (1 if wl.key_fp8 else 2) + (4 if wl.key_fp8 else 0)
        q_b = wl.D_I * (1 if wl.q_fp8 else 2) + (8 if wl.q_fp8 else 4)
        sc_bytes = wl.B * (wl.T_kv * (key_b + 4) + wl.H_I * q_b) * n_f
        achieved = sc_bytes / score_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": score_traffic(wl),
                    "kernel": f"score_splitkey_kernel<{wl.H_I},{wl.D_I},{kdt}>"}
    roofline["launches_per_step"] = nchunk * n_f
    if fused:
        roofline["fused_launches_per_step"] = n_fused * n_f
    roofline["avg_launch_ms"] = round(float(np.mean(score_ms)) / (nchunk * n_f), 4)
    # select: HBM-bound; algorithmic bytes = read each causal score once + write k indices
    # (after the fused pass the selection reads candidates, not score rows:
    # no figure then)
    sel_bytes = (pairs * 4 + n_q_total * wl.top_k * 4) * n_f
    sel_gbs = None if fused else round(sel_bytes / (float(np.mean(select_ms)) / 1e3) / 1e9, 1)
    # attention: bytes of the gathered KV rows (576 x bf16 per selected index) + Q + O
    sel_per_row = sum(min(wl.top_k, p + 1) for p in range(wl.q_pos0, wl.q_pos0 + wl.n_q)) * wl.B
    attn_bytes = (sel_per_row * wl.D_qk * 2 + n_q_total * wl.H_q * (wl.D_qk + wl.D_v) * 2) * L
    attn_gbs = attn_bytes / (float(np.mean(attn_ms)) / 1e3) / 1e9

    extra = {}
    if not args.no_allf:
        allf = tuple(1 for _ in range(L))
        plan_f = path.plan(allf)
        path.step(plan_f)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev_f = [[torch.cuda.Event(enable_timing=True) for _ in range(4 * L)] for _ in range(nchunk)]
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

    if not args.no_ceilings:
        extra["measured_ceilings"] = measured_ceilings()
        log(f"[bench] ceilings: {extra['measured_ceilings']}")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(path)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} {cpu['unit']} ({cpu['sample']})")

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
        "select_algorithmic_GBps": sel_gbs,
        "select_input": "fused candidates" if fused else "score rows",
        "attention_algorithmic_GBps": round(attn_gbs, 1),
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
