"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Each test names the plausible oracle mistake it would catch.  None of them
re-types the oracle's formula: they compare against printed values, closed
forms, brute force, invariants, or an independent library routine on a
special case.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- P-a
@pytest.mark.parametrize("d", [2, 64])
def test_printed_worked_example(d):
    """Printed SDPA example (#24): catches wrong weighting, mask polarity, lse."""
    g = _golden("sdpa_worked_example.json")
    v = np.zeros((1, 2, 1, d))
    v[0, :, 0, :2] = np.array(g["values"])
    q = np.zeros((1, 1, 1, d))
    k = _rand((1, 2, 1, d), 1)
    out, lse = oracle.attention(q, k, v, dtype="f32")
    np.testing.assert_array_equal(out[0, 0, 0, :2], g["both_sources"]["out"])
    assert lse[0, 0, 0] == pytest.approx(g["both_sources"]["lse"], abs=1e-15)
    kpm = np.array([[0, 1]], dtype=np.uint8)
    out, lse = oracle.attention(q, k, v, kpm=kpm, dtype="f32")
    np.testing.assert_array_equal(out[0, 0, 0, :2], g["second_source_excluded"]["out"])
    assert lse[0, 0, 0] == g["second_source_excluded"]["lse"]
    # the same exclusion written as an attention mask
    out2, lse2 = oracle.attention(q, k, v, attn_mask=np.array([[0, 1]], np.uint8), dtype="f32")
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)


# ---------------------------------------------------------------- P-b
def test_causal_pattern_brute_force():
    """V = I makes out the probability matrix: catches off-by-one in the
    causal test (diagonal must be allowed) and a transposed mask."""
    g = _golden("causal_pattern.json")
    T = g["T"]
    d = 8
    q = _rand((1, T, 1, d), 2)
    k = _rand((1, T, 1, d), 3)
    v = np.zeros((1, T, 1, d))
    v[0, :, 0, :T] = np.eye(T)
    out, _ = oracle.attention(q, k, v, causal=True, dtype="f32")
    P = out[0, :, 0, :T]
    allowed = np.array(g["allowed"], dtype=bool)
    assert np.all(P[~allowed] == 0.0)
    assert np.all(P[allowed] > 0.0)


@pytest.mark.parametrize("q_off,kv_off", [(0, 0), (5, 2), (3, 7), (100, 0)])
def test_causal_with_offsets_brute_force(q_off, kv_off):
    """Absolute-position causal test, checked entry by entry with python ints."""
    Tq, Tkv, d = 6, 9, 4
    q = _rand((1, Tq, 1, d), 4)
    k = _rand((1, Tkv, 1, d), 5)
    v = np.zeros((1, Tkv, 1, 16))
    v[0, :, 0, :Tkv] = np.eye(Tkv)
    out, lse = oracle.attention(q, k, v, q_off=q_off, kv_off=kv_off, causal=True, dtype="f32")
    for i in range(Tq):
        for j in range(Tkv):
            ok = kv_off + j <= q_off + i
            assert (out[0, i, 0, j] > 0) == ok
        if not any(kv_off + j <= q_off + i for j in range(Tkv)):
            assert lse[0, 0, i] == -np.inf and np.all(out[0, i, 0] == 0)


# ---------------------------------------------------------------- P-c
def test_rows_sum_to_one():
    """Row softmax is non-negative and sums to 1 (#22)."""
    B, T, H, d = 2, 37, 3, 16
    q, k = _rand((B, T, H, d), 6), _rand((B, T, H, d), 7)
    v = np.ones((B, T, H, d))
    kpm = (np.random.default_rng(8).random((B, T)) < 0.3).astype(np.uint8)
    kpm[:, 0] = 0
    out, _ = oracle.attention(q, k, v, causal=True, kpm=kpm, dtype="f32")
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- masks
def test_mask_combination_equals_key_removal():
    """kpm and attn_mask exclusions combine (#2): excluding keys must equal
    deleting them.  Catches AND instead of OR, or inverted polarity."""
    B, Tq, Tkv, H, d = 1, 5, 11, 2, 8
    q, k, v = _rand((B, Tq, H, d), 9), _rand((B, Tkv, H, d), 10), _rand((B, Tkv, H, d), 11)
    kpm = np.zeros((B, Tkv), np.uint8)
    kpm[0, [1, 4]] = 1
    am = np.zeros((Tq, Tkv), np.uint8)
    am[:, 7] = 1
    out, lse = oracle.attention(q, k, v, kpm=kpm, attn_mask=am, dtype="f32")
    keep = [j for j in range(Tkv) if j not in (1, 4, 7)]
    out2, lse2 = oracle.attention(q, k[:, keep], v[:, keep], dtype="f32")
    np.testing.assert_allclose(out, out2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


def test_masked_keys_get_exactly_zero_weight():
    """Finite garbage at masked keys must not change a single bit."""
    B, Tq, Tkv, H, d = 1, 4, 9, 1, 8
    q, k, v = _rand((B, Tq, H, d), 12), _rand((B, Tkv, H, d), 13), _rand((B, Tkv, H, d), 14)
    kpm = np.zeros((B, Tkv), np.uint8)
    kpm[0, 6:] = 1
    out, lse = oracle.attention(q, k, v, kpm=kpm, dtype="f32")
    k2, v2 = k.copy(), v.copy()
    k2[:, 6:] *= 1e3
    v2[:, 6:] = 1e3
    out2, lse2 = oracle.attention(q, k2, v2, kpm=kpm, dtype="f32")
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ---------------------------------------------------------------- P-k
@pytest.mark.parametrize("causal", [False, True])
def test_library_special_case_torch_sdpa(causal):
    """Unmasked (or plain causal), no RoPE, one block: torch's CPU float64
    scaled_dot_product_attention.  Catches a dropped 1/sqrt(d) scale or a
    transposed operand."""
    B, T, H, d = 2, 23, 3, 16
    q, k, v = _rand((B, T, H, d), 15), _rand((B, T, H, d), 16), _rand((B, T, H, d), 17)
    kpm = (np.random.default_rng(18).random((B, T)) < 0.25).astype(np.uint8)
    kpm[:, 0] = 0
    out, lse = oracle.attention(q, k, v, causal=causal, kpm=kpm, dtype="f32")
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    allow = torch.from_numpy(kpm == 0)[:, None, None, :].expand(B, 1, T, T).clone()
    if causal:
        allow &= torch.ones(T, T, dtype=torch.bool).tril()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allow)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    # lse against torch.logsumexp of the masked scores
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(~allow, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- P-l
def test_single_allowed_key_and_uniform_scores():
    """One allowed key: out = v_j exactly and lse = s_j.  Zero query: out is
    the mean of the allowed values and lse = ln(count)."""
    d = 16
    q, k, v = _rand((1, 1, 1, d), 19), _rand((1, 6, 1, d), 20), _rand((1, 6, 1, d), 21)
    kpm = np.array([[1, 1, 0, 1, 1, 1]], np.uint8)
    out, lse = oracle.attention(q, k, v, kpm=kpm, dtype="f32")
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 2, 0])
    s = float(np.dot(q[0, 0, 0], k[0, 2, 0])) / math.sqrt(d)
    assert lse[0, 0, 0] == pytest.approx(s, abs=1e-15)
    kpm = np.array([[0, 1, 0, 0, 1, 0]], np.uint8)
    out, lse = oracle.attention(np.zeros_like(q), k, v, kpm=kpm, dtype="f32")
    np.testing.assert_allclose(out[0, 0, 0], v[0, [0, 2, 3, 5], 0].mean(axis=0), atol=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(4), abs=1e-15)


def test_fully_masked_row_is_identity_partial():
    q, k, v = _rand((1, 3, 1, 4), 22), _rand((1, 3, 1, 4), 23), _rand((1, 3, 1, 4), 24)
    out, lse = oracle.attention(q, k, v, kpm=np.ones((1, 3), np.uint8), dtype="f32")
    assert np.all(out == 0) and np.all(lse == -np.inf)
    out, lse = oracle.attention(q, k[:, :0], v[:, :0], dtype="f32")
    assert out.shape == (1, 3, 1, 4) and np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- P-e / P-f
def test_merge_equals_attention_over_the_union():
    """oracle(Q, Ka u Kb) == merge(oracle(Q,Ka), oracle(Q,Kb)).  Catches any
    dropped term or wrong weight in the merge."""
    B, Tq, Tkv, H, d = 2, 7, 20, 2, 8
    q, k, v = _rand((B, Tq, H, d), 25), _rand((B, Tkv, H, d), 26), _rand((B, Tkv, H, d), 27)
    qp = np.arange(10, 10 + Tq)
    kp = np.arange(Tkv)
    full = oracle.sdpa(q, k, v, qp, kp, causal=True, dtype="f32")
    a = oracle.sdpa(q, k[:, :8], v[:, :8], qp, kp[:8], causal=True, dtype="f32")
    b = oracle.sdpa(q, k[:, 8:], v[:, 8:], qp, kp[8:], causal=True, dtype="f32")
    m = oracle.merge(*a, *b)
    np.testing.assert_allclose(m[0], full[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(m[1], full[1], atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_order_and_size_invariance(seed):
    """Online-softmax accumulation over blocks in any order and of any size
    gives the one-block result (fraction form and rescale rule)."""
    rng = np.random.default_rng(100 + seed)
    B, Tq, Tkv, H, d = 1, 9, 41, 2, 8
    q, k, v = _rand((B, Tq, H, d), 28 + seed), _rand((B, Tkv, H, d), 31 + seed), _rand((B, Tkv, H, d), 34 + seed)
    qp = np.arange(30, 30 + Tq)
    kp = np.arange(Tkv)
    kpm = (rng.random((B, Tkv)) < 0.2).astype(np.uint8)
    full = oracle.sdpa(q, k, v, qp, kp, causal=True, kpm=kpm, dtype="f32")
    cuts = np.sort(rng.choice(np.arange(1, Tkv), size=4, replace=False))
    blocks = np.split(np.arange(Tkv), cuts)
    order = rng.permutation(len(blocks))
    acc = (np.zeros_like(full[0]), np.full_like(full[1], -np.inf))
    for i in order:
        ix = blocks[i]
        part = oracle.sdpa(q, k[:, ix], v[:, ix], qp, kp[ix], causal=True, kpm=kpm[:, ix], dtype="f32")
        acc = oracle.merge(*acc, *part)
    np.testing.assert_allclose(acc[0], full[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(acc[1], full[1], atol=1e-12, rtol=0)


def test_merge_identity_and_commutativity():
    B, Tq, H, d = 1, 5, 2, 4
    oa, la = _rand((B, Tq, H, d), 40), _rand((B, H, Tq), 41)
    ob, lb = _rand((B, Tq, H, d), 42), _rand((B, H, Tq), 43)
    la[0, 0, 1] = -np.inf
    oa[0, 1, 0] = 0.0
    zero, ninf = np.zeros_like(oa), np.full_like(la, -np.inf)
    o, l = oracle.merge(oa, la, zero, ninf)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o1, l1 = oracle.merge(oa, la, ob, lb)
    o2, l2 = oracle.merge(ob, lb, oa, la)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o, l = oracle.merge(zero, ninf, zero, ninf)
    assert np.all(o == 0) and np.all(l == -np.inf)


# ---------------------------------------------------------------- P-g RoPE
def test_rope_closed_forms():
    """Pair 0 turns by exactly pos radians (theta_0 = 1) in the positive sense;
    pair t turns by base^(-2t/d) per position (RoFormer schedule).  Catches a
    sign flip, a rotate-half pairing, or a wrong exponent."""
    d, base = 16, 10000.0
    x = np.zeros((1, 1, 1, d))
    x[..., 0::2] = 1.0                                # every pair starts at (1, 0)
    for pos in [0, 1, 7, 1000, 131071]:
        y = oracle.rope_rotate(x, np.array([pos]), base)[0, 0, 0]
        assert y[0] == pytest.approx(math.cos(pos), abs=1e-12)
        assert y[1] == pytest.approx(math.sin(pos), abs=1e-12)
    y = oracle.rope_rotate(x, np.array([1]), base)[0, 0, 0]
    for t in range(d // 2):
        ang = math.atan2(y[2 * t + 1], y[2 * t])
        assert ang == pytest.approx(base ** (-2.0 * t / d), abs=1e-14)
    x = _rand((1, 3, 2, d), 44)
    np.testing.assert_array_equal(oracle.rope_rotate(x, np.zeros(3), base), x)


def test_rope_invariants():
    """Pair norms are preserved and the rotated dot product depends only on
    m - n ("Transformers and Attention" #4)."""
    d, base = 64, 10000.0
    q = _rand((1, 1, 1, d), 45)
    k = _rand((1, 1, 1, d), 46)
    y = oracle.rope_rotate(q, np.array([12345]), base)
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, q[..., 0::2] ** 2 + q[..., 1::2] ** 2, atol=1e-12)
    def dot(m, n):
        return float(np.dot(oracle.rope_rotate(q, np.array([m]), base)[0, 0, 0],
                            oracle.rope_rotate(k, np.array([n]), base)[0, 0, 0]))
    for m, n, sh in [(10, 3, 1000), (0, 0, 777), (5000, 4000, 120000)]:
        assert dot(m, n) == pytest.approx(dot(m + sh, n + sh), abs=1e-10)
    assert dot(10, 3) != pytest.approx(dot(10, 4), abs=1e-6)


def test_rope_attention_shift_invariance():
    """Attention with RoPE and causal mask is unchanged by a common shift of
    q_off and kv_off, up to the dtype rounding of the rotated operands."""
    B, T, H, d = 1, 12, 2, 16
    q, k, v = _rand((B, T, H, d), 47), _rand((B, T, H, d), 48), _rand((B, T, H, d), 49)
    a = oracle.attention(q, k, v, q_off=0, kv_off=0, causal=True, rope_base=10000.0, dtype="f32")
    b = oracle.attention(q, k, v, q_off=5000, kv_off=5000, causal=True, rope_base=10000.0, dtype="f32")
    np.testing.assert_allclose(a[0], b[0], atol=1e-5)
    np.testing.assert_allclose(a[1], b[1], atol=1e-5)
    # position 0 rotation is the identity, so rope at offset 0 with T=1 equals no rope
    c = oracle.attention(q[:, :1], k[:, :1], v[:, :1], causal=True, rope_base=10000.0, dtype="bf16")
    e = oracle.attention(q[:, :1], k[:, :1], v[:, :1], causal=True, dtype="bf16")
    np.testing.assert_array_equal(c[0], e[0])


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_matches_torch_on_float32_inputs():
    """On float32-representable inputs, direct RNE to bf16 must agree with
    torch's float32 -> bfloat16 conversion bit for bit."""
    x = np.random.default_rng(50).standard_normal(200000).astype(np.float32)
    x = np.concatenate([x, x * 1e-30, x * 1e30, np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.5 - 2 ** -8])])
    ours = R.round_to_dtype(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    assert R.round_to_dtype(np.array([1.0 + 2 ** -8]), "bf16")[0] == 1.0          # tie -> even
    assert R.round_to_dtype(np.array([1.0 + 3 * 2 ** -8]), "bf16")[0] == 1.0 + 2 ** -6
    assert R.round_to_dtype(np.array([1.0 + 2 ** -8 + 2 ** -40]), "bf16")[0] == 1.0 + 2 ** -7


# ---------------------------------------------------------------- P-h / P-i
def test_causal_pair_counts_printed():
    g = _golden("causal_pair_counts.json")
    T = g["T"]
    for key in ("contiguous", "zigzag"):
        for gpu, want in zip(("gpu0_tokens", "gpu1_tokens"), g[key]["pairs"]):
            assert oracle.allowed_pairs(g[key][gpu], range(T)) == want
    P = g["P"]
    for r, gpu in enumerate(("gpu0_tokens", "gpu1_tokens")):
        pos = oracle.local_query_positions(T, P, r, zigzag=True)
        assert sorted(pos.tolist()) == g["zigzag"][gpu]
        pos = oracle.local_query_positions(T, P, r, zigzag=False)
        assert sorted(pos.tolist()) == g["contiguous"][gpu]


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("c", [1, 2, 3])
def test_zigzag_closed_form_brute_force(P, c):
    T = 2 * P * c
    counts = {oracle.allowed_pairs(oracle.local_query_positions(T, P, r, True), range(T)) for r in range(P)}
    assert counts == {oracle.zigzag_pairs_closed_form(P, c)}
    cover = np.sort(np.concatenate([oracle.local_query_positions(T, P, r, True) for r in range(P)]))
    np.testing.assert_array_equal(cover, np.arange(T))


def test_zigzag_pairs_128k_share():
    """One rank's share of an 8-way zigzag ring at 128K: 1,073,750,016 causal
    pairs per head, checked by counting rows (not the closed form)."""
    T, P = 131072, 8
    qp = oracle.local_query_positions(T, P, 0, True)
    assert int((qp + 1).sum()) == oracle.zigzag_pairs_closed_form(P, T // (2 * P)) == 1_073_750_016


def test_ring_order_printed():
    g = _golden("ring_order.json")
    assert oracle.ring_order(g["P"], g["rank"]) == g["order"]
    assert len(oracle.ring_order(g["P"], g["rank"])) - 1 == g["transfers"]
    for P in (1, 2, 4, 8):
        for r in range(P):
            o = oracle.ring_order(P, r)
            assert o[0] == r and sorted(o) == list(range(P))
            assert all(o[i + 1] == (o[i] - 1) % P for i in range(P - 1))


# ---------------------------------------------------------------- P-j / P-m
def test_score_variance_before_scaling():
    """For iid N(0,1) coordinates var(q.k) = d (#15, section 3.2.1)."""
    d = 128
    rng = np.random.default_rng(51)
    q, k = rng.standard_normal((200000, d)), rng.standard_normal((200000, d))
    var = float(np.var(np.einsum("nd,nd->n", q, k)))
    assert var == pytest.approx(d, rel=0.02)


def test_permutation_equivariance_without_positions():
    """Set Transformer (#18): with no positions and no causal order,
    permuting keys (with their kpm entries) leaves out/lse unchanged, and
    permuting queries permutes the outputs."""
    B, Tq, Tkv, H, d = 1, 6, 10, 2, 8
    rng = np.random.default_rng(52)
    q, k, v = _rand((B, Tq, H, d), 53), _rand((B, Tkv, H, d), 54), _rand((B, Tkv, H, d), 55)
    kpm = (rng.random((B, Tkv)) < 0.3).astype(np.uint8)
    kpm[0, 0] = 0
    out, lse = oracle.attention(q, k, v, kpm=kpm, dtype="f32")
    pk = rng.permutation(Tkv)
    out2, lse2 = oracle.attention(q, k[:, pk], v[:, pk], kpm=kpm[:, pk], dtype="f32")
    np.testing.assert_allclose(out2, out, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)
    pq = rng.permutation(Tq)
    out3, lse3 = oracle.attention(q[:, pq], k, v, kpm=kpm, dtype="f32")
    np.testing.assert_array_equal(out3, out[:, pq])
    np.testing.assert_array_equal(lse3, lse[:, :, pq])


def test_fused_rope_equals_stored_bf16_rotation_then_attention():
    """Reading of the pages' silence on RoPE precision: attention with RoPE on
    bf16 inputs equals rotating, storing the result as bf16 (torch's own
    conversion here, not the oracle's rounding) and then attending without
    RoPE.  Catches an oracle that forgets to round the rotated operands."""
    B, T, H, d = 1, 64, 2, 64
    x = workloads_bf16((B, T, H, d), 60)
    y = workloads_bf16((B, T, H, d), 61)
    v = workloads_bf16((B, T, H, d), 62)
    q_off, kv_off = 70000, 69990
    qr = oracle.rope_rotate(x, q_off + np.arange(T), 10000.0)
    kr = oracle.rope_rotate(y, kv_off + np.arange(T), 10000.0)
    qs = torch.from_numpy(qr).to(torch.float32).to(torch.bfloat16).double().numpy()
    ks = torch.from_numpy(kr).to(torch.float32).to(torch.bfloat16).double().numpy()
    a = oracle.attention(x, y, v, q_off=q_off, kv_off=kv_off, causal=True, rope_base=10000.0, dtype="bf16")
    b = oracle.attention(qs, ks, v, q_off=q_off, kv_off=kv_off, causal=True, dtype="bf16")
    # identical except where float64 -> float32 -> bf16 double rounding hits a tie
    assert np.mean(np.abs(a[1] - b[1]) == 0) > 0.99
    np.testing.assert_allclose(a[1], b[1], atol=1e-4)
    np.testing.assert_allclose(a[0], b[0], atol=1e-3)


def workloads_bf16(shape, seed):
    return torch.from_numpy(_rand(shape, seed)).to(torch.float32).to(torch.bfloat16).double().numpy()


def test_rope_matches_gptj_interleaved_rotary():
    """The pairing (adjacent coordinates 2t, 2t+1) and the frequency schedule
    (theta_t = base^(-2t/d)), a reading of "Transformers and Attention" #4,
    agree with an independent implementation: the interleaved rotary
    embedding of the GPT-J model in the installed transformers package, which
    forms its angles in float32 (hence the tolerance: about 2^-24 of an angle
    of at most 255 rad).  A rotate-half pairing, a wrong exponent or a
    reversed turning sense are off by O(1)."""
    gptj = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    for d in (64, 128):
        T, H = 256, 3
        x = workloads_bf16((2, T, H, d), 71 + d)
        sincos = gptj.create_sinusoidal_positions(T, d)             # (T, d): sin | cos, float32
        sin, cos = torch.split(sincos.double(), d // 2, dim=-1)
        pos = torch.arange(T)
        ref = gptj.apply_rotary_pos_emb(torch.from_numpy(x), sin[pos][None].expand(2, T, d // 2),
                                        cos[pos][None].expand(2, T, d // 2)).numpy()
        got = oracle.rope_rotate(x, np.arange(T), 10000.0)
        norm = np.abs(x).max()
        assert np.abs(got - ref).max() <= 4e-5 * norm


def test_rope_frequency_schedule_structure():
    """The turning rates read back from rotated unit vectors (atan2, not the
    schedule's formula) start at 1 rad per position, fall geometrically (a
    constant ratio between neighbours) and pair up as theta_t *
    theta_(d/2-t) = 1/base; together these fix theta_t = base^(-2t/d)."""
    for d, base in [(64, 10000.0), (128, 10000.0), (128, 500000.0)]:
        x = np.zeros((1, 1, 1, d))
        x[..., 0::2] = 1.0
        y = oracle.rope_rotate(x, np.array([1]), base)[0, 0, 0]
        th = np.arctan2(y[1::2], y[0::2])                      # all rates are below pi
        assert th[0] == pytest.approx(1.0, abs=1e-15)
        ratios = th[1:] / th[:-1]
        np.testing.assert_allclose(ratios, ratios[0], rtol=1e-12)
        for t in range(1, d // 2):
            assert th[t] * th[d // 2 - t] == pytest.approx(1.0 / base, rel=1e-12)


def test_rotated_operand_is_the_float64_rotation_rounded_once():
    """The rotated operand the attention definition uses is the float64
    rotation rounded once to the input dtype (reading R1): identity at
    position 0, bf16-representable values, and each within half a bf16 unit
    of the exact rotation (checked against the unit of the value itself)."""
    from oracle import reference as ref
    d, base = 128, 10000.0
    x = workloads_bf16((1, 50, 3, d), 70)
    pos = np.concatenate([[0, 1, 2], np.arange(131000, 131047)])
    exact = oracle.rope_rotate(x, pos, base)
    r = ref._rotated(x, pos, base, "bf16")
    np.testing.assert_array_equal(r[:, 0], x[:, 0])
    as_bf16 = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(r, as_bf16)
    nz = exact != 0
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact[nz]))) - 7)
    assert np.all(np.abs(r[nz] - exact[nz]) <= ulp / 2)
    r32 = ref._rotated(x, pos, base, "f32")
    np.testing.assert_array_equal(r32, exact.astype(np.float32).astype(np.float64))
