"""Pins of the oracle's variants: sliding window, ALiBi bias, and decoding
over a key/value cache ("Transformers and Attention" #53, #55, #57, #58).

Each test names the mistake it would catch.  The window is checked against
array slicing (an independent statement of "keys within left/right of the
query"), ALiBi against closed-form geometric sums and torch's float64 SDPA
with an additive mask, decoding against the full causal forward (a cached
step must give the same row as attending over the whole prefix).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ------------------------------------------------------------------ window
@pytest.mark.parametrize("window,causal,q_off,kv_off", [
    ((0, 0), False, 0, 0),
    ((2, 1), False, 0, 0),
    ((-1, 3), False, 5, 3),
    ((3, -1), False, 2, 4),
    ((4, -1), True, 0, 0),
    ((1, 5), True, 7, 2),
])
def test_window_uniform_scores_is_mean_of_the_slice(window, causal, q_off, kv_off):
    """q = 0 makes every score 0, so each row averages the values of the keys
    in its window: out_i = mean(v[lo:hi]), lse_i = ln(hi - lo), with lo, hi
    from slicing positions.  Catches an off-by-one at either edge, a swapped
    left/right, or a window measured in local rather than absolute positions."""
    Tq, Tkv, d = 9, 12, 4
    q = np.zeros((1, Tq, 1, d))
    k = _rand((1, Tkv, 1, d), 1)
    v = _rand((1, Tkv, 1, d), 2)
    out, lse = oracle.attention(q, k, v, q_off=q_off, kv_off=kv_off, causal=causal, window=window, dtype="f64")
    left, right = window
    kpos = kv_off + np.arange(Tkv)
    for i in range(Tq):
        p = q_off + i
        lo_pos = -10 ** 9 if left < 0 else p - left
        hi_pos = 10 ** 9 if right < 0 else p + right
        if causal:
            hi_pos = min(hi_pos, p)
        lo = int(np.searchsorted(kpos, lo_pos, side="left"))
        hi = int(np.searchsorted(kpos, hi_pos, side="right"))
        if hi <= lo:
            assert np.all(out[0, i] == 0) and lse[0, 0, i] == -np.inf
            continue
        np.testing.assert_allclose(out[0, i, 0], v[0, lo:hi, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(hi - lo)) < 1e-13


def test_window_equals_attention_over_the_sliced_keys():
    """For each query, the windowed result equals plain attention over only
    the keys of its window (taken by slicing): catches a window that leaks
    or drops keys with random scores and RoPE at absolute positions."""
    Tq, Tkv, H, d = 6, 16, 2, 8
    q = _rand((1, Tq, H, d), 3)
    k = _rand((1, Tkv, H, d), 4)
    v = _rand((1, Tkv, H, d), 5)
    q_off, left, right = 8, 3, 2
    out, lse = oracle.attention(q, k, v, q_off=q_off, window=(left, right), rope_base=100.0, dtype="bf16")
    for i in range(Tq):
        p = q_off + i
        lo, hi = max(0, p - left), min(Tkv, p + right + 1)
        o1, l1 = oracle.sdpa(q[:, i:i + 1], k[:, lo:hi], v[:, lo:hi], [p], np.arange(lo, hi), rope_base=100.0,
                             dtype="bf16")
        np.testing.assert_allclose(out[:, i:i + 1], o1, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i:i + 1], l1, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ ALiBi
@pytest.mark.parametrize("slope", [0.5, 0.0625])
def test_alibi_causal_closed_form(slope):
    """q = 0, causal, positions 0..T-1: row i weighs key j by r^(i-j) with
    r = e^-slope, so lse_i = ln((1 - r^(i+1)) / (1 - r)) and, with one-hot
    values (V = I), out_ij = r^(i-j) (1 - r) / (1 - r^(i+1)).  Catches a
    wrong sign of the bias, a bias scaled by 1/sqrt(d), or a distance
    measured from the wrong end."""
    T, d = 10, 16
    q = np.zeros((1, T, 1, d))
    k = _rand((1, T, 1, d), 6)
    v = np.eye(T, d)[None, :, None, :]
    out, lse = oracle.attention(q, k, v, causal=True, alibi_slopes=[slope], dtype="f64")
    r = math.exp(-slope)
    for i in range(T):
        assert abs(lse[0, 0, i] - math.log((1 - r ** (i + 1)) / (1 - r))) < 1e-13
        want = np.array([r ** (i - j) * (1 - r) / (1 - r ** (i + 1)) if j <= i else 0.0 for j in range(T)])
        np.testing.assert_allclose(out[0, i, 0, :T], want, rtol=1e-12, atol=1e-15)


def test_alibi_symmetric_closed_form():
    """Non-causal: keys after the query are penalised by the same distance
    rule, so lse_i = ln(sum_{j<=i} r^(i-j) + sum_{j>i} r^(j-i)) in closed
    form.  Catches a one-sided (signed) distance."""
    T, d, slope = 9, 8, 0.3
    q = np.zeros((1, T, 1, d))
    k = _rand((1, T, 1, d), 7)
    v = _rand((1, T, 1, d), 8)
    _, lse = oracle.attention(q, k, v, alibi_slopes=[slope], dtype="f64")
    r = math.exp(-slope)
    for i in range(T):
        tot = (1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (T - 1 - i)) / (1 - r)
        assert abs(lse[0, 0, i] - math.log(tot)) < 1e-13


def test_alibi_torch_additive_mask():
    """torch's float64 SDPA with the distance penalty given as an additive
    float mask (added to the scaled scores) agrees, per head slope: pins
    where the bias enters (after 1/sqrt(d), before softmax) and that each
    head takes its own slope."""
    B, T, H, d = 1, 7, 3, 16
    q, k, v = (_rand((B, T, H, d), s) for s in (9, 10, 11))
    slopes = [0.25, 0.5, 1.0]
    out, lse = oracle.attention(q, k, v, alibi_slopes=slopes, dtype="f64")
    dist = np.abs(np.subtract.outer(np.arange(T), np.arange(T))).astype(np.float64)
    bias = torch.tensor(np.stack([-s * dist for s in slopes]))[None]           # (1, H, T, T)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=bias)
    np.testing.assert_allclose(out, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-12)


def test_alibi_zero_slope_and_shift_invariance():
    """Slope 0 is plain attention (bit-identical); the penalty depends on
    distances only, so shifting query and key positions together changes
    nothing (no RoPE)."""
    B, Tq, Tkv, H, d = 1, 5, 8, 2, 8
    q, k, v = _rand((B, Tq, H, d), 12), _rand((B, Tkv, H, d), 13), _rand((B, Tkv, H, d), 14)
    o0, l0 = oracle.attention(q, k, v, q_off=3, causal=True, dtype="f64")
    o1, l1 = oracle.attention(q, k, v, q_off=3, causal=True, alibi_slopes=[0.0, 0.0], dtype="f64")
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    oa, la = oracle.attention(q, k, v, q_off=3, kv_off=0, alibi_slopes=[0.4, 0.1], dtype="f64")
    ob, lb = oracle.attention(q, k, v, q_off=1003, kv_off=1000, alibi_slopes=[0.4, 0.1], dtype="f64")
    np.testing.assert_allclose(oa, ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ decoding
@pytest.mark.parametrize("rope_base,window_left,alibi", [
    (0.0, -1, False),
    (10000.0, -1, False),
    (500.0, 4, False),
    (10000.0, -1, True),
])
def test_decode_steps_equal_the_causal_forward(rope_base, window_left, alibi):
    """Appending one token at a time and attending with its query gives the
    same row as the causal forward over the whole prefix (#53: cached keys
    and values are exactly the ones a full pass would use).  Two sequences
    with different prompt lengths share the cache.  Catches a key rotated to
    the wrong position, an off-by-one in the cache length, a window counted
    from the wrong end, or a bias with the wrong distance."""
    B, H, d, Tcap = 2, 2, 8, 12
    prompt = [3, 6]
    steps = 5
    T = max(prompt) + steps
    q = _rand((B, T, H, d), 20)
    k = _rand((B, T, H, d), 21)
    v = _rand((B, T, H, d), 22)
    q, k, v = (oracle.round_to_dtype(x, "bf16") for x in (q, k, v))
    slopes = [0.3, 0.05] if alibi else None
    kc = np.full((B, Tcap, H, d), 7.0)          # unused slots hold garbage
    vc = np.full((B, Tcap, H, d), -3.0)
    ln = np.zeros(B, np.int64)
    for t in range(max(prompt)):                 # fill the prompts token by token
        for b in range(B):
            if t < prompt[b]:
                one = np.array([ln[b] if bb == b else Tcap for bb in range(B)])
                kc, vc, one = oracle.kv_append(kc, vc, one, k[:, t], v[:, t], rope_base=rope_base)
                ln[b] = one[b]
    assert list(ln) == prompt
    for s in range(steps):
        pos = [prompt[b] + s for b in range(B)]
        kn = np.stack([k[b, pos[b]] for b in range(B)])
        vn = np.stack([v[b, pos[b]] for b in range(B)])
        qn = np.stack([q[b, pos[b]] for b in range(B)])
        kc, vc, ln = oracle.kv_append(kc, vc, ln, kn, vn, rope_base=rope_base)
        out, lse = oracle.decode(qn, kc, vc, ln, rope_base=rope_base, window_left=window_left, alibi_slopes=slopes)
        for b in range(B):
            n = pos[b] + 1
            of, lf = oracle.attention(q[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], causal=True,
                                      rope_base=rope_base, window=(window_left, -1), alibi_slopes=slopes)
            np.testing.assert_allclose(out[b], of[0, -1], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b], lf[0, :, -1], rtol=1e-12, atol=1e-13)


def test_kv_append_full_cache_and_empty_decode():
    """A full cache row is left as it is (no write past the last slot, length
    unchanged); a row with no filled slot decodes to (0, -inf)."""
    B, Tcap, H, d = 2, 3, 1, 4
    kc = _rand((B, Tcap, H, d), 30)
    vc = _rand((B, Tcap, H, d), 31)
    ln = np.array([3, 0])
    kn, vn = _rand((B, H, d), 32), _rand((B, H, d), 33)
    kc2, vc2, ln2 = oracle.kv_append(kc, vc, ln, kn, vn)
    assert np.array_equal(kc2[0], kc[0]) and np.array_equal(vc2[0], vc[0]) and ln2[0] == 3
    assert np.array_equal(kc2[1, 0], kn[1]) and np.array_equal(vc2[1, 0], vn[1]) and ln2[1] == 1
    out, lse = oracle.decode(_rand((B, H, d), 34), kc, vc, np.array([2, 0]))
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(lse[0]))
