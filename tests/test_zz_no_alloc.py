"""sparse_attn_noalloc: the decode partials in the library's static device
scratch instead of a workspace.  Called through the C ABI, it must give the
same bytes as sparse_attn on the same inputs (and match the oracle on a few
rows), on two calls in a row -- the second with a smaller input, so stale
scratch contents from the first call cannot leak into the second -- and
allocate nothing."""
import numpy as np
import pytest
import torch

import oracle
from helpers import ATTN_ATOL, bf16_to_f64, bits, log
from long_context_sparse_idx_amd import lcsi

pytestmark = pytest.mark.gpu


def decode_inputs(B, H, n_kv, k, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, 1, H, 576, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, n_kv, 576, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    idx = np.full((B, 1, k), -1, np.int32)
    for b in range(B):
        m = min(k, n_kv)
        idx[b, 0, :m] = np.sort(rng.choice(n_kv, m, replace=False))
    return q, kv, idx


def test_noalloc_matches_sparse_attn_on_two_calls():
    for B, H, n_kv, k, seed in ((16, 64, 6000, 2048, 1), (3, 32, 2000, 700, 2)):
        log(f"[noalloc] B={B} H={H} T_kv={n_kv} top_k={k}")
        q, kv, idx = decode_inputs(B, H, n_kv, k, seed)
        dq, dkv, didx = q.cuda(), kv.cuda(), torch.from_numpy(idx).cuda()
        tau = 576 ** -0.5
        ref = torch.full((B, 1, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        d_ref = lcsi.attn_desc(dq, dkv, dkv[..., :512], ref, k, n_kv - 1, tau)
        assert lcsi.sparse_attn_ws_bytes(d_ref) > 0          # the call has partials to hold
        assert lcsi.sparse_attn_ws_bytes(d_ref) <= lcsi.LCSI_NOALLOC_SCRATCH_BYTES
        lcsi.sparse_attn(d_ref, didx)
        out = torch.full((B, 1, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        d = lcsi.attn_desc(dq, dkv, dkv[..., :512], out, k, n_kv - 1, tau)
        torch.cuda.synchronize()
        n_alloc = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        lcsi.sparse_attn_noalloc(d, didx)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == n_alloc
        assert np.array_equal(bits(out), bits(ref))
        K = bits(kv[0])
        for b in (0, B - 1):
            K = bits(kv[b])
            o = oracle.attn(bits(q[b]), K, (K, 512), idx[b], tau)
            err = np.abs(bf16_to_f64(bits(out[b])) - bf16_to_f64(o)).max()
            log(f"  sequence {b}: max abs err {err:.3e}")
            assert err <= ATTN_ATOL
