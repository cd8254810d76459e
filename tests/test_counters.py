"""The counter summaries behind the benchmark's `hbm` block
(long_context_sparse_idx_amd/counters.py) on synthetic rocprofv3 databases,
bench.py's lookup of an entry by kernel and source hash, and bench.py's
refusal of a multi-GPU run.  CPU only."""
import hashlib
import json
import os
import sqlite3
import sys

import pytest

from long_context_sparse_idx_amd import counters

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATTN = "void lcsi::(anonymous namespace)::attn_kernel<576, 512, 2, 2, true>(lcsi::AttnArgs)"
MERGE = "void lcsi::(anonymous namespace)::attn_merge_kernel<8>(lcsi::AttnArgs)"
COPY = "__amd_rocclr_copyBuffer"
SUM = "void at::native::reduce_kernel<512, 1>(...)"


def make_db(path, rows, kernels=()):
    """rows: (dispatch_id, kernel_name, counter_name, value); kernels: (name, start, end)."""
    db = sqlite3.connect(path)
    db.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, value real)")
    db.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    db.execute("create table kernels (name text, start int, end int)")
    db.executemany("insert into kernels values (?, ?, ?)", kernels)
    db.commit()
    db.close()
    return path


@pytest.fixture
def tmp_profiles(tmp_path, monkeypatch):
    monkeypatch.setattr(counters, "PROFILES", str(tmp_path))
    monkeypatch.setattr(counters, "HBM_JSON", str(tmp_path / "hbm_counters.json"))
    return tmp_path


def sha(src):
    with open(os.path.join(ROOT, "long_context_sparse_idx_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def test_short_name_strips_namespace_and_arguments():
    assert counters.short_name(ATTN) == "attn_kernel<576, 512, 2, 2, true>"
    assert counters.short_name("lcsi::(anonymous namespace)::select_kernel(lcsi::SelectArgs)") == "select_kernel"


def test_hbm_entries_scale_by_the_copy_calibration(tmp_profiles):
    # a 1 GiB copy reads back as half its bytes in FETCH_SIZE and all of them
    # in WRITE_SIZE; the read-only reduction as half
    fetch = make_db(tmp_profiles / "f.db", [
        (1, COPY, "FETCH_SIZE", 524288.0), (2, SUM, "FETCH_SIZE", 524288.0),
        (3, ATTN, "FETCH_SIZE", 1000.0), (4, MERGE, "FETCH_SIZE", 10.0), (5, ATTN, "FETCH_SIZE", 3000.0),
        (6, MERGE, "FETCH_SIZE", 30.0), (7, "some_other_kernel", "FETCH_SIZE", 99.0)])
    write = make_db(tmp_profiles / "w.db", [
        (1, COPY, "WRITE_SIZE", 1048576.0), (3, ATTN, "WRITE_SIZE", 400.0), (4, MERGE, "WRITE_SIZE", 4.0),
        (5, ATTN, "WRITE_SIZE", 600.0), (6, MERGE, "WRITE_SIZE", 6.0)])
    counters.hbm("wl", str(fetch), str(write))
    doc = json.loads((tmp_profiles / "hbm_counters.json").read_text())
    cal = doc["calibration"]["wl"]
    assert cal["fetch_factor"] == pytest.approx(2.0) and cal["write_factor"] == pytest.approx(1.0)
    assert cal["read_fetch_factor"] == pytest.approx(2.0)
    by = {e["kernel"]: e for e in doc["entries"]}
    assert set(by) == {"attn_kernel<576, 512, 2, 2, true>", "attn_merge_kernel<8>"}  # unknown kernels dropped
    a = by["attn_kernel<576, 512, 2, 2, true>"]
    assert a["dispatches"] == 2 and a["fetch_kib"] == 2000.0 and a["write_kib"] == 500.0
    assert a["bytes_per_launch"] == (2000 * 2 + 500) * 1024
    assert a["sources"] == {"attn.hip": sha("attn.hip")}
    md = (tmp_profiles / "wl_hbm_counters.md").read_text()
    assert "attn_kernel<576, 512, 2, 2, true>" in md and "FETCH_SIZE x 2.000" in md
    # a second workload keeps the first one's entries
    counters.hbm("wl2", str(fetch), str(write))
    doc = json.loads((tmp_profiles / "hbm_counters.json").read_text())
    assert {e["workload"] for e in doc["entries"]} == {"wl", "wl2"}


def test_hbm_needs_the_copy_dispatch(tmp_profiles):
    fetch = make_db(tmp_profiles / "f.db", [(1, ATTN, "FETCH_SIZE", 1.0)])
    write = make_db(tmp_profiles / "w.db", [(1, ATTN, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        counters.hbm("wl", str(fetch), str(write))


def test_trace_summarises_durations(tmp_profiles):
    db = make_db(tmp_profiles / "t.db", [], kernels=[(ATTN, 0, 30000), (ATTN, 100, 50100), (COPY, 0, 1000000)])
    out = tmp_profiles / "trace.md"
    counters.trace(str(out), "title", "cmd", str(db))
    text = out.read_text()
    assert "| `attn_kernel<576, 512, 2, 2, true>` | 2 | 0.080 | 0.0400 |" in text
    assert "other kernels" in text and "| 1 | 1.0 |" in text


def test_bench_uses_an_entry_only_while_its_sources_match(tmp_profiles, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    path = tmp_profiles / "hbm_counters.json"
    entry = {"workload": "wl", "kernel": "attn_kernel<576, 512, 2, 2, true>", "dispatches": 2,
             "fetch_kib": 1.0, "write_kib": 1.0, "bytes_per_launch": 3072, "sources": {"attn.hip": sha("attn.hip")}}
    path.write_text(json.dumps({"entries": [entry]}))
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(path))
    assert bench.counter_entry("wl", "attn_kernel")["bytes_per_launch"] == 3072
    assert bench.counter_entry("wl", "attn_kernel", ", true>") is not None
    assert bench.counter_entry("wl", "attn_kernel", ", false>") is None
    assert bench.counter_entry("other", "attn_kernel") is None
    entry["sources"]["attn.hip"] = "0" * 64   # measured on other sources
    path.write_text(json.dumps({"entries": [entry]}))
    assert bench.counter_entry("wl", "attn_kernel") is None


def test_bench_stage_bytes_sum_every_variant_per_call(tmp_profiles, monkeypatch):
    """A stage's bytes per call: every template variant of its kernels (a
    decode group's attention launches with and without the previous layer's
    merge, and its one merge launch) over the calls, one per primary launch."""
    sys.path.insert(0, ROOT)
    import bench
    path = tmp_profiles / "hbm_counters.json"
    src = {"attn.hip": sha("attn.hip")}
    es = [{"workload": "wl", "kernel": "attn_kernel<576, 512, 4, 2, true, true>", "dispatches": 7,
           "bytes_per_launch": 1000, "sources": src},
          {"workload": "wl", "kernel": "attn_kernel<576, 512, 4, 2, true, false>", "dispatches": 1,
           "bytes_per_launch": 600, "sources": src},
          {"workload": "wl", "kernel": "attn_merge_kernel", "dispatches": 1, "bytes_per_launch": 400,
           "sources": src}]
    path.write_text(json.dumps({"entries": es}))
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(path))
    st = bench.hbm_stage_for("wl", "attn_kernel", ("attn_merge_kernel",), 0.001)
    assert st["bytes_per_call"] == (7 * 1000 + 600 + 400) // 8
    assert st["GBps"] == pytest.approx(1000.0 / 1e-6 / 1e9)
    assert bench.hbm_stage_for("wl", "select_filter_kernel", (), 0.001) is None
    es[1]["sources"] = {"attn.hip": "0" * 64}   # one variant measured on other sources
    path.write_text(json.dumps({"entries": es}))
    assert bench.hbm_stage_for("wl", "attn_kernel", ("attn_merge_kernel",), 0.001) is None


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus N with N > 1 exits with a message (the library has no
    multi-GPU mode); checked before anything touches a GPU."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_mfma_summary_derives_clock_and_busy_fraction(tmp_profiles):
    """Busy cycles per SIMD over active cycles per XCD, and the clock from
    the active cycles over the dispatch's duration."""
    K = "void lcsi::(anonymous namespace)::score_prefill_kernel<64, 128, 0, true>(lcsi::ScoreArgs)"
    db = make_db(tmp_profiles / "m.db", [
        (1, K, "SQ_INSTS_VALU_MFMA_BF16", 4.0e8), (1, K, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0e10),
        (1, K, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.5e7), (1, K, "GRBM_GUI_ACTIVE", 8 * 2.0e7)],
        kernels=[(K, 0, 10_000_000)])   # 10 ms
    out = tmp_profiles / "mfma.md"
    counters.mfma(str(out), "title", "cmd", str(db))
    text = out.read_text()
    assert "| `score_prefill_kernel<64, 128, 0, true>` | 1 | 10.000 | 4e+08 | 1.024e+13 | 1.5e+07 | 2e+07 | 2.00 | 75 % |" in text
