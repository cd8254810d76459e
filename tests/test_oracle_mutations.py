"""The oracle's pins catch plausible slips: each case below plants one
mistake in a copy of the C oracle (never in the working tree), builds it
into a temporary library, and runs the pin suite against that build
(LCSI_ORACLE_LIB); the suite must fail.  An unmodified copy built the same
way must pass, which checks the harness itself."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lcsi_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (what the slip is, text in the oracle, what it becomes)
MUTANTS = [
    ("ReLU dropped", "double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    ("head weight dropped", "score += (double)w[h] * relu;", "score += relu;"),
    ("query operand transposed", "dot += qd[h * D + d] * kd[d];", "dot += qd[d * H + h] * kd[d];"),
    ("last causal key (the diagonal) skipped",
     "for (int64_t s = 0; s < n; s++) {\n        for (int d = 0; d < D; d++) {",
     "for (int64_t s = 0; s < n - 1; s++) {\n        for (int d = 0; d < D; d++) {"),
    ("-0 score kept as -0", "if (f == 0.0f)\n            f = 0.0f;", ""),
    ("fp8 key scale dropped", "kd[d] = oracle_fp8e4m3_to_double(kr[d]) * (double)k_scale[s];",
     "kd[d] = oracle_fp8e4m3_to_double(kr[d]);"),
    ("fp8 query scale dropped", "oracle_fp8e4m3_to_double(((const uint8_t *)q)[i]) * (double)q_scale[i / D]",
     "oracle_fp8e4m3_to_double(((const uint8_t *)q)[i])"),
    ("fp8 exponent bias off by one", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("fp8 subnormal scale wrong", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("bf16 decode shifted", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("bf16 rounding ties away from zero", "double r = nearbyint(q);", "double r = floor(q + 0.5);"),
    ("tie rule reversed (higher position first)", "return (x->i > y->i) - (x->i < y->i);",
     "return (x->i < y->i) - (x->i > y->i);"),
    ("value order reversed", "if (x->v > y->v)\n        return -1;", "if (x->v < y->v)\n        return -1;"),
    ("indices left in score order", "qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);", ""),
    ("padding 0 instead of -1", "for (int64_t j = m; j < k; j++)\n        out[j] = -1;",
     "for (int64_t j = m; j < k; j++)\n        out[j] = 0;"),
    ("softmax scale dropped", "logit[j] = tau * dot;", "logit[j] = dot;"),
    ("softmax normaliser wrong", "denom += p;", "denom += 1.0;"),
]


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, LCSI_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def _build(text: str, d: str) -> str:
    os.makedirs(d, exist_ok=True)
    src, lib = os.path.join(d, "oracle.c"), os.path.join(d, "oracle.so")
    with open(src, "w") as f:
        f.write(text)
    oracle.compile_source(src, lib)
    return lib


def test_every_planted_slip_fails_the_pins(tmp_path):
    base = open(SRC).read()
    for name, old, new in MUTANTS:
        assert base.count(old) == 1, f"{name}: the oracle text to mutate is not there exactly once"

    def run(case):
        i, (name, old, new) = case
        lib = _build(base.replace(old, new, 1), str(tmp_path / f"m{i}"))
        return name, _run_pins(lib)

    control = _run_pins(_build(base, str(tmp_path / "control")))
    assert control.returncode == 0, "unmodified oracle copy fails its pins:\n" + control.stdout[-2000:]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(run, enumerate(MUTANTS)))
    missed = [name for name, r in results if r.returncode == 0]
    assert not missed, f"pins did not catch: {missed}"
