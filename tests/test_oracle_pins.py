"""Pins for the CPU oracle: each check compares it with something other than
itself -- library conversions, exact integer arithmetic, brute force by the
rank definition, a library sort, dense softmax attention from torch, closed
forms and hand-derived fixtures under tests/golden/.

A plausible slip anywhere in the oracle (a dropped ReLU or weight, a wrong
sign, a transposed operand, an off-by-one causal bound, a reversed tie rule,
an unsorted result, a dropped -1 skip, a wrong rounding) fails at least one
test here.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x):
    """float array -> bf16 bit patterns (uint16) via torch's RNE cast."""
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b):
    return torch.from_numpy(np.asarray(b, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


# ------------------------------------------------------------------ decoding

def test_bf16_decode_matches_torch_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits_to_f64(pats)
    got = np.array([oracle.bf16_to_double(int(p)) for p in pats])
    r = ref
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])


def test_fp8_decode_matches_torch_and_spec():
    allb = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(allb).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8e4m3_to_double(int(b)) for b in allb])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # format facts: largest finite 448, smallest subnormal 2^-9, 1.0 = 0x38
    assert oracle.fp8e4m3_to_double(0x7E) == 448.0
    assert oracle.fp8e4m3_to_double(0x01) == 2.0 ** -9
    assert oracle.fp8e4m3_to_double(0x38) == 1.0
    assert oracle.fp8e4m3_to_double(0xB8) == -1.0
    assert math.isnan(oracle.fp8e4m3_to_double(0x7F))


def _bf16_rne_exact(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even to 8 significant bits (normal range)."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    q = abs(x) / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


def test_double_to_bf16_rounding():
    # hand cases: halfway ties go to the even neighbour
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.double_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.double_to_bf16(-2.0) == 0xC000
    assert oracle.double_to_bf16(2.0 ** -133) == 0x0001
    assert oracle.double_to_bf16(1.5 * 2.0 ** -133) == 0x0002
    assert oracle.double_to_bf16(0.4 * 2.0 ** -133) == 0x0000
    assert oracle.double_to_bf16((2 - 2.0 ** -7) * 2.0 ** 127) == 0x7F7F
    assert oracle.double_to_bf16(2.0 ** 128 * 0.999999) == 0x7F80
    assert oracle.double_to_bf16(0.46211715726000974) == 0x3EED
    # random doubles against an exact rational rounding
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(400) * np.exp(rng.uniform(-30, 30, 400))
    for x in xs:
        want = float(_bf16_rne_exact(Fraction(float(x))))
        got = bits_to_f64([oracle.double_to_bf16(float(x))])[0]
        assert got == want, (x, got, want)


# --------------------------------------------------------------------- score

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_score_select_golden_fixture():
    g = _golden("score_select_tiny.json")
    q = bf16_bits(np.array(g["q"], np.float32))[None]
    w = np.array(g["w"], np.float32)[None]
    keys = bf16_bits(np.array(g["keys"], np.float32))
    s, idx = oracle.score_select(q, w, keys, [5], 4)
    assert s[0].tolist() == g["scores_p5"]
    assert idx[0].tolist() == g["topk_p5"]["4"]
    for kk, want in g["topk_p5"].items():
        _, idx = oracle.score_select(q, w, keys, [5], int(kk))
        assert idx[0].tolist() == want
    s, idx = oracle.score_select(q, w, keys, [1], 3)
    assert s[0, :2].tolist() == g["scores_p1"]
    assert idx[0].tolist() == g["topk3_p1"]


def test_score_below_fp32_range_is_stored_as_plus_zero():
    """A negative score too small for fp32 rounds to zero; the oracle stores
    +0 (sign bit clear), never -0, so a score row compares bit for bit with
    one whose -0 results are folded (the reading that -0 counts as +0).
    Here the only product is 2^-133 * 2^-133 (the smallest bf16 subnormal
    squared) under a weight of -1: the exact score is -2^-266."""
    q = np.zeros((1, 1, 8), np.uint16)
    keys = np.zeros((2, 8), np.uint16)
    q[0, 0, 0] = 0x0001
    keys[:, 0] = 0x0001
    w = np.array([[-1.0]], np.float32)
    s, idx = oracle.score_select(q, w, keys, [1], 1)
    assert s[0, 0] == 0.0 and s[0, 1] == 0.0
    assert not np.signbit(s[0, :2]).any()
    assert idx[0].tolist() == [0]


def _int_inputs(rng, R, H, D, N):
    q = rng.integers(-8, 9, (R, H, D)).astype(np.float32)
    k = rng.integers(-8, 9, (N, D)).astype(np.float32)
    w = (2.0 ** rng.integers(-3, 1, (R, H))).astype(np.float32)
    return q, k, w


def test_score_integer_exact():
    """Integer q,k in [-8,8] and power-of-two w: the exact score is a
    rational with small numerator, representable in fp32; the oracle must
    reproduce it bit for bit.  Exact reference via Python integers."""
    rng = np.random.default_rng(2)
    R, H, D, N = 5, 6, 16, 40
    q, k, w = _int_inputs(rng, R, H, D, N)
    pos = np.array([0, 1, 17, 38, 39])
    s, _ = oracle.score_select(bf16_bits(q), w, bf16_bits(k), pos, 8)
    qi, ki = q.astype(np.int64), k.astype(np.int64)
    for r in range(R):
        for t in range(pos[r] + 1):
            exact = Fraction(0)
            for h in range(H):
                dot = int(sum(int(qi[r, h, d]) * int(ki[t, d]) for d in range(D)))
                exact += Fraction(float(w[r, h])) * max(dot, 0)
            assert s[r, t] == np.float32(float(exact)), (r, t)


def test_score_single_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(3)
    D, N = 64, 70
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((N, D)).astype(np.float32)
    qb, kb = bf16_bits(q), bf16_bits(k)
    s, _ = oracle.score_select(qb, np.ones((1, 1), np.float32), kb, [N - 1], 4)
    dots = bits_to_f64(kb) @ bits_to_f64(qb[0, 0])
    want = np.maximum(dots, 0.0).astype(np.float32)
    # library dot product sums in another order: allow one fp32 ulp
    assert np.all(np.abs(s[0] - want) <= np.spacing(np.abs(want)))
    assert np.array_equal(s[0] == 0, dots <= 0)


def test_score_weights_scale_exactly_and_keep_indices():
    rng = np.random.default_rng(4)
    R, H, D, N = 4, 8, 32, 90
    q = bf16_bits(rng.standard_normal((R, H, D)) / 8)
    k = bf16_bits(rng.standard_normal((N, D)) / 8)
    w = rng.uniform(0, 1, (R, H)).astype(np.float32)
    pos = np.array([10, 40, 70, 89])
    s1, i1 = oracle.score_select(q, w, k, pos, 16)
    s2, i2 = oracle.score_select(q, 2 * w, k, pos, 16)
    assert np.array_equal(s2, 2 * s1)
    assert np.array_equal(i1, i2)


def test_score_is_causal():
    """Row p depends on keys 0..p only, and the diagonal key p counts."""
    rng = np.random.default_rng(5)
    R, H, D, N = 1, 4, 16, 30
    q = bf16_bits(rng.standard_normal((R, H, D)))
    k = rng.standard_normal((N, D)).astype(np.float32)
    p = 12
    s1, i1 = oracle.score_select(q, np.ones((R, H), np.float32), bf16_bits(k), [p], 5)
    k2 = k.copy()
    k2[p + 1:] = 100.0  # keys after p must not matter
    s2, i2 = oracle.score_select(q, np.ones((R, H), np.float32), bf16_bits(k2), [p], 5)
    assert np.array_equal(s1[0, :p + 1], s2[0, :p + 1])
    assert np.array_equal(i1, i2)
    k3 = k.copy()
    k3[p] = 50.0 * np.sign(np.asarray(bits_to_f64(q[0, 0]), np.float32) + 1e-9)
    _, i3 = oracle.score_select(q, np.ones((R, H), np.float32), bf16_bits(k3), [p], 1)
    assert i3[0, 0] == p  # a dominant diagonal key is selected


def test_fp8_keys_equal_bf16_keys_with_same_values():
    """fp8 keys decode exactly; with a power-of-two scale the decoded key is
    exactly a bf16 value, so scores must equal the bf16-key scores."""
    rng = np.random.default_rng(6)
    R, H, D, N = 3, 4, 32, 50
    q = bf16_bits(rng.standard_normal((R, H, D)) / 8)
    w = rng.uniform(0, 1, (R, H)).astype(np.float32)
    k8 = torch.from_numpy(rng.standard_normal((N, D)).astype(np.float32) * 4).to(
        torch.float8_e4m3fn)
    scale = (2.0 ** rng.integers(-4, 3, N)).astype(np.float32)
    kval = k8.to(torch.float64).numpy() * scale[:, None]
    pos = np.array([5, 30, 49])
    s8, i8 = oracle.score_select(q, w, k8.view(torch.uint8).numpy(), pos, 7, k_scale=scale)
    sb, ib = oracle.score_select(q, w, bf16_bits(kval.astype(np.float32)), pos, 7)
    assert np.array_equal(s8, sb)
    assert np.array_equal(i8, ib)
    # a non-power-of-two scale multiplies the key, not the score rounding
    scale3 = np.full(N, 3.0, np.float32)
    s3, _ = oracle.score_select(q, w, k8.view(torch.uint8).numpy(), pos, 7, k_scale=scale3)
    s1, _ = oracle.score_select(q, w, k8.view(torch.uint8).numpy(), pos, 7,
                                k_scale=np.ones(N, np.float32))
    assert np.allclose(s3, 3 * s1, rtol=2 ** -23, atol=0)


def test_fp8_queries_equal_bf16_queries_with_same_values():
    """fp8 queries with a per-head scale decode to value * scale: with
    power-of-two scales that is exactly a bf16 value, so scores must equal the
    bf16-query scores bit for bit.  Distinct scales per head catch a scale
    applied to the wrong head (or per row instead of per head)."""
    rng = np.random.default_rng(16)
    R, H, D, N = 3, 5, 32, 60
    k8 = torch.from_numpy(rng.standard_normal((N, D)).astype(np.float32) * 4).to(torch.float8_e4m3fn)
    kscale = (2.0 ** rng.integers(-5, -1, N)).astype(np.float32)
    q8 = torch.from_numpy(rng.standard_normal((R, H, D)).astype(np.float32) * 8).to(torch.float8_e4m3fn)
    qscale = (2.0 ** rng.integers(-6, 0, (R, H))).astype(np.float32)
    w = rng.uniform(0, 1, (R, H)).astype(np.float32)
    pos = np.array([7, 33, 59])
    qval = q8.to(torch.float64).numpy() * qscale[:, :, None]
    kb = k8.view(torch.uint8).numpy()
    s8, i8 = oracle.score_select(q8.view(torch.uint8).numpy(), w, kb, pos, 9, k_scale=kscale, q_scale=qscale)
    sb, ib = oracle.score_select(bf16_bits(qval.astype(np.float32)), w, kb, pos, 9, k_scale=kscale)
    assert np.array_equal(s8, sb)
    assert np.array_equal(i8, ib)
    # the per-head scale acts like a factor on that head's weight (exact for
    # powers of two, and ReLU commutes with a positive factor)
    s1, _ = oracle.score_select(q8.view(torch.uint8).numpy(), w * qscale, kb, pos, 9, k_scale=kscale,
                                q_scale=np.ones((R, H), np.float32))
    assert np.array_equal(s8, s1)


# -------------------------------------------------------------------- select

def rank_definition(row, k):
    """s is chosen iff fewer than k entries beat it (larger value, or equal
    value at a lower position).  -0.0 == +0.0 under the IEEE compare."""
    n = len(row)
    chosen = []
    for s in range(n):
        beats = sum(1 for j in range(n)
                    if row[j] > row[s] or (row[j] == row[s] and j < s))
        if beats < k:
            chosen.append(s)
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_rank_definition_with_ties(seed):
    rng = np.random.default_rng(10 + seed)
    n = int(rng.integers(1, 200))
    k = int(rng.integers(1, 40))
    row = rng.integers(-3, 4, n).astype(np.float32)  # heavy ties
    row[rng.random(n) < 0.2] = -0.0
    row[rng.random(n) < 0.2] = 0.0
    got = oracle.select(row[None], [n], k)[0].tolist()
    assert got == rank_definition(row.tolist(), k)


@pytest.mark.parametrize("seed", range(4))
def test_select_matches_library_sort(seed):
    rng = np.random.default_rng(20 + seed)
    n, k = 3000, 257
    row = rng.standard_normal(n).astype(np.float32)
    row[::17] = row[3]  # some exact ties
    order = np.lexsort((np.arange(n), -row.astype(np.float64)))
    want = np.sort(order[:k])
    got = oracle.select(row[None], [n], k)[0]
    assert np.array_equal(got, want)


def test_select_special_rows():
    k = 8
    assert oracle.select(np.full((1, 50), 1.5, np.float32), [50], k)[0].tolist() == list(range(k))
    inc = np.arange(50, dtype=np.float32)[None]
    assert oracle.select(inc, [50], k)[0].tolist() == list(range(42, 50))
    assert oracle.select(inc, [5], k)[0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    # only the first n entries of a row count
    row = np.zeros((1, 20), np.float32)
    row[0, 15] = 9.0
    assert 15 not in oracle.select(row, [10], 3)[0].tolist()
    # -0.0 and +0.0 tie: the lower position wins
    row = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert oracle.select(row, [3], 1)[0].tolist() == [0]
    row = np.array([[0.0, -0.0, -1.0]], np.float32)
    assert oracle.select(row, [3], 1)[0].tolist() == [0]


# ----------------------------------------------------------------- attention

def test_attn_golden_fixture():
    g = _golden("attn_tiny.json")
    q = bf16_bits(np.array(g["q"], np.float32))[None]
    K = bf16_bits(np.array(g["K"], np.float32))
    V = bf16_bits(np.array(g["V"], np.float32))
    for c in g["cases"]:
        idx = np.array([c["idx"]], np.int32)
        out = oracle.attn(q, K, V, idx, g["tau"])
        assert bits_to_f64(out[0, 0]).tolist() == c["out"], c


def _dense_masked_attention(q, K, V, masks, tau):
    """torch float64 softmax attention with a boolean key mask per row."""
    qd = torch.from_numpy(bits_to_f64(q))          # [R, H, Dqk]
    Kd = torch.from_numpy(bits_to_f64(K))          # [N, Dqk]
    Vd = torch.from_numpy(bits_to_f64(V))          # [N, Dv]
    logits = tau * torch.einsum("rhd,nd->rhn", qd, Kd)
    m = torch.from_numpy(masks)[:, None, :]
    logits = logits.masked_fill(~m, float("-inf"))
    p = torch.softmax(logits, dim=-1)
    return torch.einsum("rhn,nd->rhd", p, Vd).numpy()


def _bf16_close(got_bits, want_f64):
    """Equal after bf16 rounding up to one bf16 ulp (the two sides sum in
    different orders, so a value near a rounding boundary may differ)."""
    got = bits_to_f64(got_bits)
    want = bits_to_f64(bf16_bits(want_f64.astype(np.float32)))
    ulp = np.maximum(np.abs(want), 2.0 ** -126) * 2.0 ** -7
    return np.all(np.abs(got - want) <= ulp)


def test_attn_all_causal_keys_is_dense_causal_attention():
    rng = np.random.default_rng(30)
    N, H, Dqk, Dv = 48, 3, 16, 8
    K = bf16_bits(rng.standard_normal((N, Dqk)))
    V = bf16_bits(rng.standard_normal((N, Dv)))
    pos = np.array([0, 1, 7, 30, 47])
    q = bf16_bits(rng.standard_normal((len(pos), H, Dqk)))
    k = 64  # >= every row's causal length
    idx = np.full((len(pos), k), -1, np.int32)
    for r, p in enumerate(pos):
        idx[r, :p + 1] = np.arange(p + 1)
    tau = 1 / math.sqrt(Dqk)
    out = oracle.attn(q, K, V, idx, tau)
    causal = np.arange(N)[None, :] <= pos[:, None]
    assert _bf16_close(out, _dense_masked_attention(q, K, V, causal, tau))


def test_attn_matches_dense_masked_to_index_set_and_is_permutation_invariant():
    rng = np.random.default_rng(31)
    N, H, Dqk, Dv, k = 100, 4, 32, 16, 12
    Kfull = bf16_bits(rng.standard_normal((N, Dqk)))
    pos = np.array([20, 60, 99])
    q = bf16_bits(rng.standard_normal((len(pos), H, Dqk)))
    idx = np.stack([np.sort(rng.choice(p + 1, k, replace=False)) for p in pos]).astype(np.int32)
    tau = 0.125
    # MLA-style shared row: V is the first Dv columns of the same rows
    out = oracle.attn(q, Kfull, (Kfull, Dv), idx, tau)
    mask = np.zeros((len(pos), N), bool)
    for r in range(len(pos)):
        mask[r, idx[r]] = True
    want = _dense_masked_attention(q, Kfull, np.ascontiguousarray(Kfull[:, :Dv]), mask, tau)
    assert _bf16_close(out, want)
    perm = idx[:, rng.permutation(k)]
    out2 = oracle.attn(q, Kfull, (Kfull, Dv), perm, tau)
    assert _bf16_close(out2, bits_to_f64(out))
    # -1 padding is skipped
    pad = np.concatenate([idx, np.full((len(pos), 5), -1, np.int32)], axis=1)
    out3 = oracle.attn(q, Kfull, (Kfull, Dv), pad, tau)
    assert np.array_equal(out3, out)


def test_attn_single_index_returns_that_row():
    rng = np.random.default_rng(32)
    N, H, Dqk, Dv = 40, 5, 16, 24
    K = bf16_bits(rng.standard_normal((N, Dqk)))
    V = bf16_bits(rng.standard_normal((N, Dv)))
    q = bf16_bits(rng.standard_normal((3, H, Dqk)))
    idx = np.array([[3], [17], [39]], np.int32)
    out = oracle.attn(q, K, V, idx, 0.3)
    for r in range(3):
        for h in range(H):
            assert np.array_equal(out[r, h], V[idx[r, 0]])


# --------------------------------------------------------------- layer group

def test_layer_group_f_and_s_layers():
    rng = np.random.default_rng(40)
    N, HI, DI, Hq, D, k = 64, 4, 16, 2, 16, 8
    pos = np.array([3, 20, 63])
    R = len(pos)
    pattern = [1, 0, 0, 0, 1, 0]
    f_layers = [dict(q=bf16_bits(rng.standard_normal((R, HI, DI))),
                     w=rng.uniform(0, 1, (R, HI)).astype(np.float32),
                     keys=bf16_bits(rng.standard_normal((N, DI))))
                for _ in range(2)]
    attn_layers = [dict(q=bf16_bits(rng.standard_normal((R, Hq, D))),
                        K=bf16_bits(rng.standard_normal((N, D))),
                        V=bf16_bits(rng.standard_normal((N, D))), tau=0.25)
                   for _ in pattern]
    idxs, outs = oracle.layer_group(pattern, f_layers, attn_layers, pos, k)
    # F layers equal a direct indexer call; S layers reuse the nearest F
    _, i0 = oracle.score_select(f_layers[0]["q"], f_layers[0]["w"], f_layers[0]["keys"], pos, k)
    _, i4 = oracle.score_select(f_layers[1]["q"], f_layers[1]["w"], f_layers[1]["keys"], pos, k)
    for l in range(4):
        assert np.array_equal(idxs[l], i0)
    assert np.array_equal(idxs[4], i4) and np.array_equal(idxs[5], i4)
    assert not np.array_equal(i0, i4)
    # every layer runs its own attention on the shared set
    for l, idx in enumerate(idxs):
        a = attn_layers[l]
        assert np.array_equal(outs[l], oracle.attn(a["q"], a["K"], a["V"], idx, a["tau"]))
    assert not np.array_equal(outs[1], outs[2])
    # all-F equals one indexer call per layer
    f_all = [f_layers[0]] * 6
    idxs_f, _ = oracle.layer_group([1] * 6, f_all, attn_layers, pos, k)
    assert all(np.array_equal(i, i0) for i in idxs_f)
    with pytest.raises(ValueError):
        oracle.layer_group([0, 1], f_layers[:1], attn_layers[:2], pos, k)
