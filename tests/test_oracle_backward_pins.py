"""Pins of the fp64 backward oracle (``oracle.sdpa_backward``).

Each test names the mistake it would catch.  None re-types the oracle's
formula: they compare against central finite differences of the forward
oracle, an independent route to the probabilities (V = I), invariants of the
softmax, a closed form and torch's float64 autograd on a special case.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, g, **kw):
    out, _ = oracle.attention(q, k, v, **kw)
    return float((out * g).sum())


def _fd_grad(x, f, h=1e-6):
    gx = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy()
        xm = x.copy()
        xp[i] += h
        xm[i] -= h
        gx[i] = (f(xp) - f(xm)) / (2 * h)
    return gx


@pytest.mark.parametrize("case", [
    dict(causal=False),
    dict(causal=True, q_off=3, kv_off=0),
    dict(causal=True, q_off=2, kv_off=1, rope_base=100.0),
    dict(causal=False, kpm=np.array([[0, 1, 0, 0, 1, 0]], np.uint8), rope_base=50.0),
    dict(causal=True, q_off=4, kv_off=0, attn_mask=(np.arange(30).reshape(5, 6) % 4 == 1).astype(np.uint8)),
    dict(causal=False, q_off=2, kv_off=0, window=(2, 1)),
    dict(causal=True, q_off=3, kv_off=1, window=(3, -1), alibi_slopes=[0.5, 0.125], rope_base=100.0),
    dict(causal=False, alibi_slopes=[0.25, 1.0]),
])
def test_finite_differences(case):
    """Central differences of the forward definition in float64 (exact
    rotation, no rounding): catches a dropped row-sum term, a sign or scale
    error, transposed dS, a wrong RoPE back-rotation, gradients leaking
    through masked pairs or pairs outside a window, an ALiBi penalty left
    out of P."""
    B, Tq, Tkv, H, d = 1, 5, 6, 2, 4
    q = _rand((B, Tq, H, d), 1)
    k = _rand((B, Tkv, H, d), 2)
    v = _rand((B, Tkv, H, d), 3)
    g = _rand((B, Tq, H, d), 4)
    kw = dict(dtype="f64", **case)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, **kw)
    fq = _fd_grad(q, lambda x: _loss(x, k, v, g, **kw))
    fk = _fd_grad(k, lambda x: _loss(q, x, v, g, **kw))
    fv = _fd_grad(v, lambda x: _loss(q, k, x, g, **kw))
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, f, rtol=1e-7, atol=1e-8)


def test_dv_from_the_probabilities_of_the_forward():
    """dv = P^T dout with P read off the forward oracle through V = I
    (out = P when the values are one-hot): an independent route to P;
    catches a transposed P or a wrong causal alignment in the backward."""
    T, d = 6, 8
    q = _rand((1, T, 1, d), 5)
    k = _rand((1, T, 1, d), 6)
    eye = np.eye(T, d)[None, :, None, :]
    P, _ = oracle.attention(q, k, eye, causal=True, q_off=1, kv_off=0, dtype="f64")
    P = P[0, :, 0, :T]                                             # (Tq, Tkv)
    g = _rand((1, T, 1, d), 7)
    v = _rand((1, T, 1, d), 8)
    _, _, dv = oracle.attention_backward(q, k, v, g, causal=True, q_off=1, kv_off=0, dtype="f64")
    np.testing.assert_allclose(dv[0, :, 0, :], P.T @ g[0, :, 0, :], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1])
def test_key_gradients_sum_to_zero(seed):
    """Shifting every key by the same vector adds a row constant to each
    row's allowed scores, which softmax ignores, so sum_j dk_j = 0 for any
    mask (without RoPE): catches a missing or wrong row-sum term in dS."""
    B, T, H, d = 2, 7, 2, 8
    q = _rand((B, T, H, d), seed)
    k = _rand((B, T, H, d), seed + 10)
    v = _rand((B, T, H, d), seed + 20)
    g = _rand((B, T, H, d), seed + 30)
    kpm = (np.arange(B * T).reshape(B, T) % 3 == 2).astype(np.uint8)
    _, dk, _ = oracle.attention_backward(q, k, v, g, causal=True, kpm=kpm, dtype="f64")
    assert np.abs(dk.sum(axis=1)).max() < 1e-12


def test_single_allowed_key():
    """A row that sees one key has P = 1 there: out = v_j whatever q and k
    are, so dq = dk = 0 and dv_j = dout_i exactly."""
    d = 8
    q = _rand((1, 1, 1, d), 11)
    k = _rand((1, 3, 1, d), 12)
    v = _rand((1, 3, 1, d), 13)
    g = _rand((1, 1, 1, d), 14)
    kpm = np.array([[1, 0, 1]], np.uint8)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, kpm=kpm, dtype="f64")
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv[0, 1], g[0, 0])
    assert np.all(dv[0, 0] == 0) and np.all(dv[0, 2] == 0)


def test_fully_masked_row_contributes_nothing():
    """A query row with no allowed key (out = 0, lse = -inf) has no
    gradient path: its dq is 0 and removing it changes no dk or dv."""
    d = 8
    q = _rand((1, 3, 1, d), 21)
    k = _rand((1, 4, 1, d), 22)
    v = _rand((1, 4, 1, d), 23)
    g = _rand((1, 3, 1, d), 24)
    am = np.zeros((3, 4), np.uint8)
    am[1, :] = 1
    dq, dk, dv = oracle.attention_backward(q, k, v, g, attn_mask=am, dtype="f64")
    assert np.all(dq[0, 1] == 0)
    keep = [0, 2]
    dq2, dk2, dv2 = oracle.attention_backward(q[:, keep], k, v, g[:, keep], attn_mask=am[keep], dtype="f64")
    np.testing.assert_allclose(dk, dk2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dv, dv2, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_library_special_case_torch_autograd(causal):
    """No mask, no RoPE: torch's float64 SDPA backward on the CPU agrees to
    1e-12 (a cross-check of the oracle only)."""
    B, T, H, d = 2, 9, 3, 16
    q = _rand((B, T, H, d), 31)
    k = _rand((B, T, H, d), 32)
    v = _rand((B, T, H, d), 33)
    g = _rand((B, T, H, d), 34)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, causal=causal, dtype="f64")
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.tensor(g.transpose(0, 2, 1, 3)))
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)


def test_share_gradients_equal_full_sequence_gradients():
    """A rank's share (its query rows against every key at absolute
    positions) gives the same dk, dv as the full sequence with dout zero on
    the other rows, and the same dq on its rows: catches position and
    indexing mistakes in the share form the ring check relies on."""
    T, H, d, P = 16, 2, 8, 2
    q = _rand((1, T, H, d), 41)
    k = _rand((1, T, H, d), 42)
    v = _rand((1, T, H, d), 43)
    g = _rand((1, T, H, d), 44)
    rows = oracle.local_query_positions(T, P, 0, True)
    kw = dict(causal=True, rope_base=1000.0, dtype="bf16")
    dq_s, dk_s, dv_s = oracle.sdpa_backward(q[:, rows], k, v, g[:, rows], rows, np.arange(T), **kw)
    g_full = np.zeros_like(g)
    g_full[:, rows] = g[:, rows]
    dq_f, dk_f, dv_f = oracle.sdpa_backward(q, k, v, g_full, np.arange(T), np.arange(T), **kw)
    np.testing.assert_allclose(dq_s, dq_f[:, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk_s, dk_f, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv_s, dv_f, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("case", [
    dict(causal=False, kp=0.0, rope=0.0, q_off=0, kv_off=0),
    dict(causal=True, kp=0.0, rope=10000.0, q_off=40, kv_off=0),
    dict(causal=True, kp=0.3, rope=500.0, q_off=5, kv_off=20),    # rows before the first key: lse = -inf
    dict(causal=False, kp=0.5, rope=0.0, q_off=0, kv_off=0),
])
def test_key_block_gradients_equal_the_full_backward(case):
    """``key_block_gradients`` (a key block's dk, dv from dout, the operands
    and the forward's out and lse) against the rows of ``sdpa_backward``'s
    full chain rule, for key subsets in any order, padded keys included.
    Catches a delta summed over the block's keys only, a normalisation other
    than the full row's lse, a missing back-rotation of dk, and a mask taken
    for the wrong keys."""
    B, Tq, Tkv, H, d = 2, 37, 53, 2, 16
    rng = np.random.default_rng(3000 + Tq + int(case["rope"]) + int(10 * case["kp"]))
    q, k, v, g = (_rand(s, 300 + i) for i, s in enumerate([(B, Tq, H, d), (B, Tkv, H, d), (B, Tkv, H, d),
                                                            (B, Tq, H, d)]))
    kpm = (rng.random((B, Tkv)) < case["kp"]).astype(np.uint8) if case["kp"] else None
    qpos, kpos = case["q_off"] + np.arange(Tq), case["kv_off"] + np.arange(Tkv)
    kw = dict(causal=case["causal"], kpm=kpm, rope_base=case["rope"], dtype="f32")
    out, lse = oracle.sdpa(q, k, v, qpos, kpos, **kw)
    rdq, rdk, rdv = oracle.sdpa_backward(q, k, v, g, qpos, kpos, **kw)
    for rows in (np.arange(Tkv), rng.permutation(Tkv)[:11], np.array([0, Tkv - 1, 7])):
        dk, dv = oracle.key_block_gradients(q, k, v, g, out, lse, qpos, kpos, rows, **kw)
        sk = max(np.abs(rdk).max(), 1e-30)
        sv = max(np.abs(rdv).max(), 1e-30)
        assert np.abs(dk - rdk[:, rows]).max() <= 1e-10 * sk
        assert np.abs(dv - rdv[:, rows]).max() <= 1e-10 * sv


def test_key_block_gradients_finite_differences():
    """Central finite differences of the forward oracle's loss with respect to
    two listed key rows (causal, offsets, RoPE, key padding): the block
    gradient is the derivative of the whole attention, not of the block's
    own softmax."""
    B, Tq, Tkv, H, d = 1, 9, 12, 1, 4
    q, k, v, g = (_rand(s, 400 + i) for i, s in enumerate([(B, Tq, H, d), (B, Tkv, H, d), (B, Tkv, H, d),
                                                            (B, Tq, H, d)]))
    kpm = np.zeros((B, Tkv), dtype=np.uint8)
    kpm[0, 5] = 1
    kw = dict(q_off=6, kv_off=0, causal=True, kpm=kpm, rope_base=100.0, dtype="f64")
    qpos, kpos = 6 + np.arange(Tq), np.arange(Tkv)
    out, lse = oracle.sdpa(q, k, v, qpos, kpos, causal=True, kpm=kpm, rope_base=100.0, dtype="f64")
    rows = np.array([2, 9])
    dk, dv = oracle.key_block_gradients(q, k, v, g, out, lse, qpos, kpos, rows, causal=True, kpm=kpm,
                                        rope_base=100.0, dtype="f64")
    fk = _fd_grad(k, lambda x: _loss(q, x, v, g, **kw))
    fv = _fd_grad(v, lambda x: _loss(q, k, x, g, **kw))
    assert np.abs(dk - fk[:, rows]).max() <= 1e-6 * np.abs(fk).max()
    assert np.abs(dv - fv[:, rows]).max() <= 1e-6 * np.abs(fv).max()
