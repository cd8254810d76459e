"""The attention checks can tell a wrong index set from rounding (oracle
only, no GPU).  At the decode and prefill shapes the outputs are small
(|O| ~ 0.04, largest ~0.2 per row), so the absolute bound 2e-2 alone barely
separates a set that lost a tile of indices from a correct one; the
row-relative diagnostic asserted beside it (max |gpu - oracle| / max |oracle|
per row, bound ATTN_ROW_REL) must be exceeded, in every row, by the oracle's
own output when one 32-index tile of a 2048-index set is left out -- a
mistake a kernel that mishandles a tile would make."""
import numpy as np
import pytest
import torch

import oracle
from helpers import ATTN_ROW_REL, attn_row_rel, bits


@pytest.mark.parametrize("tile", [0, 17, 63])
def test_a_dropped_tile_exceeds_the_row_bound(tile):
    g = torch.Generator().manual_seed(30 + tile)
    T_kv, H, rows, k = 6000, 16, 4, 2048
    q = torch.randn(rows, H, 576, generator=g).to(torch.bfloat16)
    kv = torch.randn(T_kv, 576, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(tile)
    p0 = T_kv - rows
    idx = np.stack([np.sort(rng.choice(p0 + t + 1, k, replace=False)) for t in range(rows)]).astype(np.int32)
    K = bits(kv)
    tau = 576 ** -0.5
    full = oracle.attn(bits(q), K, (K, 512), idx, tau)
    cut = idx.copy()
    cut[:, 32 * tile:32 * tile + 32] = -1         # one tile of the set left out
    part = oracle.attn(bits(q), K, (K, 512), cut, tau)
    rel = attn_row_rel(part, full)
    assert rel.min() > 1.5 * ATTN_ROW_REL, rel
    # and the same set evaluated twice is exact (the diagnostic is 0)
    assert attn_row_rel(full, full).max() == 0.0
