"""Randomised GPU top-k against the oracle's selection, byte for byte.

Seeded random cases (shape, k, score distribution) drawn so that every tier
of the selection gets work: the LDS row path, the sampled-threshold pass, and
for few long rows the segment filter with the final select in registers, in
the workspace lists, or on the row itself (a list past its slots), the
brute-force rank of a small last radix bin, and heavy ties at the k-th value.
Each case logs its seed, so a failure can be rerun alone."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_idx_amd import lcsi
from helpers import log
from test_select_bitexact import run_select

pytestmark = pytest.mark.gpu

N_CASES = 60


def scores(rng, R, n, kind):
    if kind == "normal":
        return rng.standard_normal((R, n)).astype(np.float32)
    if kind == "ties":          # few distinct values: the k-th value is heavily tied
        card = int(rng.integers(2, 40))
        return rng.integers(0, card, (R, n)).astype(np.float32) * np.float32(0.25)
    if kind == "plateau":       # a top plateau of some percent of the row
        x = rng.standard_normal((R, n)).astype(np.float32)
        x[rng.random((R, n)) < rng.uniform(0.001, 0.08)] = 7.0
        return x
    if kind == "mixture":       # two clusters far apart (wide key range)
        x = rng.standard_normal((R, n)).astype(np.float32)
        far = rng.random((R, n)) < 0.02
        x[far] = (1e4 + rng.standard_normal(int(far.sum()))).astype(np.float32)
        return x
    if kind == "recent":        # positional bias towards the end of the row
        x = rng.standard_normal((R, n)).astype(np.float32)
        x += np.linspace(0.0, rng.uniform(0.5, 4.0), n, dtype=np.float32)[None, :]
        return x
    if kind == "signs":         # both signs and zeros of both signs
        x = rng.standard_normal((R, n)).astype(np.float32)
        z = rng.random((R, n)) < 0.1
        x[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
        return x
    raise ValueError(kind)


KINDS = ["normal", "ties", "plateau", "mixture", "recent", "signs"]


def draw(case):
    rng = np.random.default_rng(zlib.crc32(f"select-random-{case}".encode()))
    path = case % 3
    if path == 0:      # few long rows (decode-like): the two-kernel path
        B, T_q = int(rng.integers(1, 9)), int(rng.integers(1, 3))
        T_kv = int(rng.integers(32768, 400000))
    elif path == 1:    # one workgroup per row, sampled threshold
        B, T_q = 1, int(rng.integers(130, 200))
        T_kv = int(rng.integers(17000, 60000))
    else:              # rows in LDS
        B, T_q = int(rng.integers(1, 3)), int(rng.integers(2, 40))
        T_kv = int(rng.integers(300, 16384))
    q_pos0 = T_kv - T_q - int(rng.integers(0, T_kv // 4))  # rows may end before the key buffer does
    k = int(rng.choice([1, 2, 7, 64, 300, 1000, 1500, 2047, 2048]))  # the library's top-k cap is 2048
    kind = KINDS[int(rng.integers(0, len(KINDS)))]
    return rng, B, T_q, T_kv, q_pos0, k, kind


@pytest.mark.parametrize("case", range(N_CASES))
def test_select_matches_oracle_on_random_rows(case):
    rng, B, T_q, T_kv, q_pos0, k, kind = draw(case)
    log(f"[select-random] case={case} kind={kind} B={B} T_q={T_q} T_kv={T_kv} q_pos0={q_pos0} k={k}")
    S = scores(rng, B * T_q, T_kv, kind)
    g = run_select(S, B, T_q, T_kv, q_pos0, k)
    n = np.array([q_pos0 + t + 1 for _ in range(B) for t in range(T_q)], np.int64)
    r = oracle.select(S, n, k)
    bad = np.nonzero((g != r).any(axis=1))[0]
    assert bad.size == 0, f"case {case} ({kind}): rows {bad[:5]} differ; first: gpu {g[bad[0]][:8]} oracle {r[bad[0]][:8]}"
