"""Host logic of the F/S layer search (long_context_sparse_idx_amd/search.py)
and the oracle's overlap count, checked on the CPU against brute force and
hand-worked cases; plus the idx_overlap entry point's argument checks (no
launch)."""
import ctypes
import itertools

import numpy as np
import pytest

import oracle
from long_context_sparse_idx_amd import lcsi
from long_context_sparse_idx_amd.search import best_pattern, coverage, greedy_pattern, sources


def test_oracle_overlap_counts_match_python_sets():
    rng = np.random.default_rng(1)
    R, k = 30, 16
    a = np.full((R, k), -1, np.int32)
    b = np.full((R, k), -1, np.int32)
    for r in range(R):
        na, nb = rng.integers(0, k + 1, 2)
        a[r, :na] = np.sort(rng.choice(40, na, replace=False))
        b[r, :nb] = np.sort(rng.choice(40, nb, replace=False))
    want = [len({int(x) for x in a[r] if x >= 0} & {int(y) for y in b[r] if y >= 0}) for r in range(R)]
    assert oracle.overlap_counts(a, b).tolist() == want
    assert oracle.overlap_counts(a, a).tolist() == [int((a[r] >= 0).sum()) for r in range(R)]


def test_sources_and_coverage_by_hand():
    assert sources([1, 0, 0, 1, 0]) == [0, 0, 0, 3, 3]
    with pytest.raises(ValueError):
        sources([0, 1])
    M = np.array([[1.0, 0.5, 0.2],
                  [0.6, 1.0, 0.7],
                  [0.1, 0.8, 1.0]])
    assert coverage(M, [1, 0, 0]) == pytest.approx((1 + 0.6 + 0.1) / 3)
    assert coverage(M, [1, 1, 0]) == pytest.approx((1 + 1 + 0.8) / 3)
    assert coverage(M, [1, 1, 1]) == pytest.approx(1.0)


def brute_force_best(M, n_f):
    L = M.shape[0]
    best = -1.0
    for rest in itertools.combinations(range(1, L), n_f - 1):
        pat = [1 if (l == 0 or l in rest) else 0 for l in range(L)]
        best = max(best, coverage(M, pat))
    return best


def test_greedy_finds_one_f_per_block_of_similar_layers():
    """Layers in blocks that select the same sets (overlap 1) and nothing
    across blocks: the optimum keeps exactly the first layer of each block,
    and the greedy walk finds it."""
    blocks = [0, 0, 0, 1, 1, 2, 2, 2, 2, 3]
    L = len(blocks)
    M = np.array([[1.0 if blocks[i] == blocks[j] else 0.0 for j in range(L)] for i in range(L)])
    pat = greedy_pattern(M, 4)
    assert pat == (1, 0, 0, 1, 0, 1, 0, 0, 0, 1) == best_pattern(M, 4)
    assert coverage(M, pat) == pytest.approx(1.0) == pytest.approx(brute_force_best(M, 4))


@pytest.mark.parametrize("seed", range(6))
def test_exact_search_matches_brute_force_and_bounds_the_greedy(seed):
    """Overlaps that decay with layer distance (the random-walk generator's
    shape), or arbitrary ones: the dynamic programme reaches the brute-force
    optimum; the greedy walk keeps layer 0 and exactly n_f F layers and
    never beats the optimum (it need not reach it)."""
    rng = np.random.default_rng(seed)
    L, n_f = 9, 3 + seed % 3
    if seed % 2:
        M = rng.uniform(0, 1, (L, L))
        np.fill_diagonal(M, 1.0)
    else:
        pos = np.concatenate([[0.0], np.cumsum(rng.uniform(0.5, 1.5, L - 1))])
        M = np.exp(-0.3 * np.abs(pos[:, None] - pos[None, :]))
    opt = brute_force_best(M, n_f)
    best = best_pattern(M, n_f)
    assert best[0] == 1 and sum(best) == n_f
    assert coverage(M, best) == pytest.approx(opt, abs=1e-12)
    pat = greedy_pattern(M, n_f)
    assert pat[0] == 1 and sum(pat) == n_f
    assert coverage(M, pat) <= opt + 1e-12


def test_idx_overlap_argument_checks():
    FAKE = 1 << 20
    f = lcsi.lib.idx_overlap
    p = ctypes.c_void_p
    assert f(None, 64, 8, p(FAKE), 64, 8, 2, 8, 8, p(FAKE), None) == lcsi.LCSI_EINVAL
    assert f(p(FAKE), 64, 8, p(FAKE), 64, 8, 2, 8, 8, None, None) == lcsi.LCSI_EINVAL
    assert f(p(FAKE), -1, 8, p(FAKE), 64, 8, 2, 8, 8, p(FAKE), None) == lcsi.LCSI_EINVAL
    assert f(p(FAKE), 64, 8, p(FAKE), 64, 8, 0, 8, 8, p(FAKE), None) == lcsi.LCSI_EINVAL
    assert f(p(FAKE), 64, 8, p(FAKE), 64, 8, 2, 8, 4096, p(FAKE), None) == lcsi.LCSI_EUNSUPPORTED
    assert f(p(FAKE + 2), 64, 8, p(FAKE), 64, 8, 2, 8, 8, p(FAKE), None) == lcsi.LCSI_EALIGN
    assert f(p(FAKE), 64, 8, p(FAKE), 64, 8, 2, 8, 8, p(FAKE + 1), None) == lcsi.LCSI_EALIGN
