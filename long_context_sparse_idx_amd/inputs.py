"""Seeded synthetic inputs for the five workloads (shared by tests, smoke and
the benchmark; holds none of the method's arithmetic).

Every tensor is drawn from its own ``torch.Generator`` seeded from
``(seed, tensor name, layer, chunk)``; fp32 draws are cast to bf16 by
round-to-nearest-even.  The same call on the same device type returns the
same bytes.  Large tensors are drawn on the GPU in row chunks of a fixed size
so peak temporary memory stays bounded; the oracle gets host copies of the
rows it checks, so both sides consume identical bytes.

Workload shapes follow the pages' regimes (long-context prefill at 32K and
200K, decode at 131K, 1M context); the pages print no prompt data, so these
seeded inputs stand in for them.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

_CHUNK_ELEMS = 1 << 26  # elements drawn per generator chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # sequences
    T_q: int               # query rows per call (chunk size; 1 for decode)
    q_pos0: int            # absolute position of the first query row
    n_q: int               # total query rows per sequence over all chunks
    T_kv: int              # keys present (full length for the last chunk)
    pattern: tuple         # 1 = F layer, 0 = S layer
    H_I: int
    D_I: int
    top_k: int
    key_fp8: bool
    H_q: int
    D_qk: int
    D_v: int
    kv_shared: bool        # V = first D_v columns of the D_qk-wide KV row
    q_I_scale: float       # q_I ~ N(0,1) * q_I_scale
    k_I_scale: float       # k_I ~ N(0,1) * k_I_scale
    w_dist: str            # "uniform" (U(0, w_scale)) or "normal" (N(0,1))
    w_scale: float
    layer_noise: float     # per-layer q = q_0 + noise * eps_l (0: independent)
    seed: int = 0
    q_fp8: bool = False    # indexer queries quantised to e4m3 per (token, head) (needs key_fp8)
    layer_walk: bool = False  # per-layer q = q_0 + noise * (eps_1 + ... + eps_l): a random walk

    @property
    def n_layers(self):
        return len(self.pattern)

    @property
    def n_f(self):
        return sum(self.pattern)

    def chunks(self):
        """(q_pos0, T_q, T_kv) of each call that covers the n_q query rows."""
        out = []
        p = self.q_pos0
        end = self.q_pos0 + self.n_q
        while p < end:
            tq = min(self.T_q, end - p)
            out.append((p, tq, p + tq if self.T_q > 1 else self.T_kv))
            p += tq
        return out


def _fsss(L):
    return tuple(1 if l % 4 == 0 else 0 for l in range(L))


WORKLOADS = {
    # T=2048 causal, 1 sequence, 4 layers FSSS; indexer 4x64; top-64;
    # 8 query heads over one shared KV head of dim 128 (separate K and V).
    "tiny": Workload("tiny", 1, 2048, 0, 2048, 2048, _fsss(4), 4, 64, 64, False,
                     8, 128, 128, False, 1 / 8, 1 / 8, "uniform", 1.0, 0.0),
    # T=32768 prefill, FSSS; indexer 64x128 ~N(0,1)/sqrt(128), w ~U(0,1)/8;
    # top-2048; 64 heads over a 576-wide KV row (V = first 512 columns);
    # per-layer q = q_0 + 0.3 * noise.
    "prefill32k": Workload("prefill32k", 1, 32768, 0, 32768, 32768, _fsss(4), 64, 128,
                           2048, False, 64, 576, 512, True, 128 ** -0.5, 128 ** -0.5,
                           "uniform", 1 / 8, 0.3),
    # T=200000 in 8192-query chunks against resident keys, FSSS;
    # 32 heads over 576/512 KV; N(0,1)/8 indexer inputs, w ~U(0,1).
    "prefill200k": Workload("prefill200k", 1, 8192, 0, 200000, 200000, _fsss(4), 64, 128,
                            2048, False, 32, 576, 512, True, 1 / 8, 1 / 8,
                            "uniform", 1.0, 0.0),
    # decode: 32 sequences, one new token at position 131072 (131073 keys);
    # 8 layers FSSSFSSS; all inputs N(0,1).
    "decode131k": Workload("decode131k", 32, 1, 131072, 1, 131073, _fsss(8), 64, 128,
                           2048, False, 64, 576, 512, True, 1.0, 1.0, "normal", 1.0, 0.0),
    # 1M context, fp8 e4m3 keys with a per-token fp32 scale; 12 layers with
    # F at {0,3,4,8}.  (i) a 4096-query prefill chunk ending at 1M ...
    "prefill1m": Workload("prefill1m", 1, 4096, 1048576 - 4096, 4096, 1048576,
                          tuple(1 if l in (0, 3, 4, 8) else 0 for l in range(12)),
                          64, 128, 2048, True, 64, 576, 512, True, 1 / 8, 1 / 8,
                          "uniform", 1.0, 0.0),
    # ... and (ii) batch-8 decode at position 1M.
    "decode1m": Workload("decode1m", 8, 1, 1048576, 1, 1048577,
                         tuple(1 if l in (0, 3, 4, 8) else 0 for l in range(12)),
                         64, 128, 2048, True, 64, 576, 512, True, 1 / 8, 1 / 8,
                         "uniform", 1.0, 0.0),
}


# fp8 x fp8 variants: the same shapes with the indexer queries quantised to
# e4m3 per (token, head) as well (the keys of the 200K variant become fp8 too).
WORKLOADS["prefill1m_q8"] = dataclasses.replace(WORKLOADS["prefill1m"], name="prefill1m_q8", q_fp8=True)
WORKLOADS["decode1m_q8"] = dataclasses.replace(WORKLOADS["decode1m"], name="decode1m_q8", q_fp8=True)
WORKLOADS["prefill200k_q8"] = dataclasses.replace(WORKLOADS["prefill200k"], name="prefill200k_q8",
                                                  key_fp8=True, q_fp8=True)


# Layer-pattern search input: 12 indexer layers whose queries drift as a
# random walk (q_l = q_{l-1} + 0.3 eps_l), so near layers select similar
# positions and far ones less so; keys and weights shared by the layers.
WORKLOADS["search32k"] = dataclasses.replace(
    WORKLOADS["prefill32k"], name="search32k", pattern=tuple(1 if l % 4 == 0 else 0 for l in range(12)),
    layer_walk=True)


def _seed(*parts) -> int:
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _draw(shape, kind, scale, device, *seed_parts, out_dtype=torch.bfloat16):
    """Fill a tensor of ``shape`` with N(0,1)*scale or U(0,1)*scale draws,
    chunk by chunk along dim 0 (each chunk has its own seeded generator)."""
    out = torch.empty(shape, dtype=out_dtype, device=device)
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(-1, 1)
    row = flat.shape[1]
    rows_per = max(1, _CHUNK_ELEMS // max(row, 1))
    for c, r0 in enumerate(range(0, flat.shape[0], rows_per)):
        r1 = min(flat.shape[0], r0 + rows_per)
        g = torch.Generator(device=device)
        g.manual_seed(_seed(*seed_parts, c))
        if kind == "normal":
            x = torch.randn((r1 - r0, row), generator=g, device=device, dtype=torch.float32)
        else:
            x = torch.rand((r1 - r0, row), generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[r0:r1].copy_(x)
        del x
    return out


def indexer_inputs(wl: Workload, layer: int, device, n_rows: Optional[int] = None):
    """q_I [B, n_q, H_I, D_I] bf16 (or, for q_fp8 workloads, fp8 bytes as uint8
    with q_scale [B, n_q, H_I] fp32), k_I [B, T_kv, D_I] (bf16, or fp8 bytes as
    uint8 with k_scale [B, T_kv] fp32), w [B, n_q, H_I] fp32.

    Layer-dependent: with ``layer_noise`` > 0, q_I = q_0 + noise * eps_layer
    and k_I, w are shared by all layers (so adjacent-layer index sets can
    overlap); otherwise every layer draws its own q_I, k_I and w.
    """
    n_q = wl.n_q if n_rows is None else n_rows
    B, H, D = wl.B, wl.H_I, wl.D_I
    shared = wl.layer_noise > 0
    kl = 0 if shared else layer
    q = _q_with_noise(wl, "q_I", (B * n_q, H, D), wl.q_I_scale, layer, device,
                      out_dtype=torch.float32 if wl.q_fp8 else torch.bfloat16)
    q_scale = None
    if wl.q_fp8:
        # fp8 e4m3 queries: per-(token, head) scale = max|q| / 448 (a zero
        # head gets 1), then q / scale cast to e4m3 (input preparation)
        amax = q.abs().amax(dim=2)
        q_scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (q / q_scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        q_scale = q_scale.view(B, n_q, H).contiguous()
    q = q.view(B, n_q, H, D)
    w = _draw((B * n_q, H), wl.w_dist, wl.w_scale, device, wl.seed, wl.name, "w", kl,
              out_dtype=torch.float32).view(B, n_q, H)
    if not wl.key_fp8:
        k = _draw((B * wl.T_kv, D), "normal", wl.k_I_scale, device, wl.seed, wl.name,
                  "k_I", kl).view(B, wl.T_kv, D)
        return dict(q=q, k=k, k_scale=None, w=w, q_scale=q_scale)
    # fp8 e4m3 keys: per-token scale = max|k| / 448 (a zero row gets 1), then
    # k / scale cast to e4m3 (input preparation, not part of the method).
    kf = _draw((B * wl.T_kv, D), "normal", wl.k_I_scale, device, wl.seed, wl.name,
               "k_I", kl, out_dtype=torch.float32)
    amax = kf.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    k8 = (kf / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    del kf
    return dict(q=q, k=k8.view(B, wl.T_kv, D), k_scale=scale.view(B, wl.T_kv).contiguous(),
                w=w, q_scale=q_scale)


def _q_with_noise(wl, name, shape, scale, layer, device, out_dtype=torch.bfloat16):
    if wl.layer_noise > 0:
        q = _draw(shape, "normal", scale, device, wl.seed, wl.name, name, 0,
                  out_dtype=torch.float32)
        for j in (range(1, layer + 1) if wl.layer_walk else ([layer] if layer > 0 else [])):
            eps = _draw(shape, "normal", scale, device, wl.seed, wl.name, name + "_eps",
                        j, out_dtype=torch.float32)
            q.add_(eps, alpha=wl.layer_noise)
            del eps
        return q.to(out_dtype)
    return _draw(shape, "normal", scale, device, wl.seed, wl.name, name, layer, out_dtype=out_dtype)


def attn_inputs(wl: Workload, layer: int, device, n_rows: Optional[int] = None):
    """Main-attention inputs of one layer: Q [B, n_q, H_q, D_qk] bf16 and
    either kv [B, T_kv, D_qk] (V = first D_v columns) or separate k, v."""
    n_q = wl.n_q if n_rows is None else n_rows
    B = wl.B
    q = _q_with_noise(wl, "Q", (B * n_q, wl.H_q, wl.D_qk), 1.0, layer, device)
    q = q.view(B, n_q, wl.H_q, wl.D_qk)
    if wl.kv_shared:
        kv = _draw((B * wl.T_kv, wl.D_qk), "normal", 1.0, device, wl.seed, wl.name, "KV",
                   layer).view(B, wl.T_kv, wl.D_qk)
        return dict(q=q, k=kv, v=kv[..., :wl.D_v])
    k = _draw((B * wl.T_kv, wl.D_qk), "normal", 1.0, device, wl.seed, wl.name, "K",
              layer).view(B, wl.T_kv, wl.D_qk)
    v = _draw((B * wl.T_kv, wl.D_v), "normal", 1.0, device, wl.seed, wl.name, "V",
              layer).view(B, wl.T_kv, wl.D_v)
    return dict(q=q, k=k, v=v)


def sm_scale(wl: Workload) -> float:
    """Softmax temperature: 1/sqrt(D_qk) (the pages do not fix it)."""
    return wl.D_qk ** -0.5
