"""idx_overlap (index-set overlap per query row) against the oracle's plain
set intersection, exactly; and the layer-search statistics computed from GPU
overlaps equal the ones from the oracle's counts."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from helpers import log
from long_context_sparse_idx_amd import inputs, lcsi
from long_context_sparse_idx_amd.search import all_f_index_sets, best_pattern, coverage, greedy_pattern, overlap_matrix

pytestmark = pytest.mark.gpu


def random_lists(B, T, k, universe, rng):
    out = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = int(rng.choice([0, 1, k // 2, k - 1, k, rng.integers(0, k + 1)]))
            n = min(n, universe)
            out[b, t, :n] = np.sort(rng.choice(universe, n, replace=False))
    return out


@pytest.mark.parametrize("k,universe", [(7, 12), (64, 100), (2048, 3000), (2048, 200000)])
def test_overlap_counts_match_oracle(k, universe):
    log(f"[overlap] k={k} universe={universe}")
    rng = np.random.default_rng(k + universe)
    B, T = 3, 37
    a = random_lists(B, T, k, universe, rng)
    b = random_lists(B, T, k, universe, rng)
    b[0, :5] = a[0, :5]                       # identical rows
    got = lcsi.idx_overlap(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy()
    want = oracle.overlap_counts(a.reshape(-1, k), b.reshape(-1, k)).reshape(B, T)
    assert np.array_equal(got, want)


def test_overlap_on_strided_cache_slots():
    """Rows read through slot views of a larger cache (row and batch strides
    larger than k)."""
    rng = np.random.default_rng(3)
    B, T, k = 2, 20, 256
    cache = torch.full((3, B, T + 4, k), -1, dtype=torch.int32)
    cache[0, :, :T] = torch.from_numpy(random_lists(B, T, k, 1000, rng))
    cache[2, :, :T] = torch.from_numpy(random_lists(B, T, k, 1000, rng))
    c = cache.cuda()
    got = lcsi.idx_overlap(c[0, :, :T], c[2, :, :T]).cpu().numpy()
    want = oracle.overlap_counts(cache[0, :, :T].reshape(-1, k).numpy(),
                                 cache[2, :, :T].reshape(-1, k).numpy()).reshape(B, T)
    assert np.array_equal(got, want)


def test_search_statistics_from_gpu_and_oracle_counts_agree():
    """All-F index sets of a small random-walk workload: the overlap matrix
    from the GPU counts equals the one from the oracle's counts, so the
    searched patterns agree too; near layers overlap more than far ones."""
    wl = dataclasses.replace(inputs.WORKLOADS["search32k"], name="search4k", n_q=4096, T_q=4096, T_kv=4096)
    sets = all_f_index_sets(wl)
    M = overlap_matrix(sets)
    host = [s.cpu().numpy().reshape(-1, wl.top_k) for s in sets]
    L = len(sets)
    valid = [float((h >= 0).sum()) for h in host]
    Mo = np.eye(L)
    for l in range(L):
        for m in range(l + 1, L):
            c = float(oracle.overlap_counts(host[l], host[m]).sum())
            Mo[l, m], Mo[m, l] = c / valid[l], c / valid[m]
    assert np.allclose(M, Mo, rtol=0, atol=1e-12)
    assert greedy_pattern(M, 3) == greedy_pattern(Mo, 3)
    assert best_pattern(M, 3) == best_pattern(Mo, 3)
    adj = np.mean([M[l + 1, l] for l in range(L - 1)])
    far = np.mean([M[l + 6, l] for l in range(L - 6)])
    log(f"  mean overlap: adjacent {adj:.3f}, 6 apart {far:.3f}; greedy {greedy_pattern(M, 3)} "
        f"{coverage(M, greedy_pattern(M, 3)):.3f}, best {best_pattern(M, 3)} {coverage(M, best_pattern(M, 3)):.3f}")
    assert adj > far
