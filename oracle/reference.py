"""Plain float64 reference of the attention forward and its ring-share pieces.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
blocked, fused or reordered: scores are materialised in full, softmax is the
two-pass definition, and the ring share is computed as the local query rows
against every key at its absolute position (no ring is emulated).
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# dtype rounding
# --------------------------------------------------------------------------
def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` ("f32" or "bf16") with
    round-to-nearest-even, returning them widened back to float64.

    bf16 keeps 8 significant bits.  The rounding is done directly on the
    float64 bit pattern (bit 45 is the last kept mantissa bit), so there is no
    double rounding through float32 for normal numbers; values below the
    bf16 normal range (|x| < 2^-126, never drawn here) go through float32.
    Used for the reading that rotated q and k are rounded to the input dtype
    before the dot product (RoPE applied to stored bf16 tensors).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = np.ascontiguousarray(x).view(np.uint64).copy()
    keep = np.uint64(45)
    lsb = (u >> keep) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    r = ((u + half + lsb) >> keep) << keep
    out = r.view(np.float64).reshape(x.shape)
    tiny = np.abs(x) < 2.0 ** -126
    if np.any(tiny):
        t32 = x[tiny].astype(np.float32).view(np.uint32).astype(np.uint64)
        t32 = ((t32 + np.uint64(0x7FFF) + ((t32 >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
        out = out.copy()
        out[tiny] = t32.astype(np.uint32).view(np.float32).astype(np.float64)
    return out


# --------------------------------------------------------------------------
# rotary position embedding
# --------------------------------------------------------------------------
def rope_frequencies(d: int, base: float) -> np.ndarray:
    """theta_t = base^(-2t/d) for pair t = 0 .. d/2-1 (RoFormer's schedule;
    the digest entry #4 of "Transformers and Attention" only states that an
    even-dimensional vector is split into coordinate pairs, each rotated by a
    positional angle).  Pinned against the interleaved rotary embedding of
    the GPT-J model in the transformers package (base 10000)."""
    t = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * t / d)


def rope_rotate(x, pos, base: float) -> np.ndarray:
    """Rotate adjacent coordinate pairs (2t, 2t+1) of x[..., T, H, d] by the
    angle pos[T] * theta_t ("Transformers and Attention", #4 RoFormer and #30:
    sine/cosine rotations).  Pair (x0, x1) becomes
    (x0 cos a - x1 sin a, x0 sin a + x1 cos a).  float64 throughout."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[:, None] * rope_frequencies(d, base)[None, :]          # (T, d/2)
    c = np.cos(ang)[:, None, :]                                      # (T, 1, d/2) -> broadcast over heads
    s = np.sin(ang)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# --------------------------------------------------------------------------
# scaled dot-product attention, plain definition
# --------------------------------------------------------------------------
def _rotated(x, pos, base: float, dtype: str) -> np.ndarray:
    """Rotated operand as the attention sees it: the float64 rotation
    (``rope_rotate``) rounded once to the input dtype, as if the rotation had
    been applied to the stored tensors ("Transformers and Attention" #4:
    coordinate pairs turned by a positional angle; #31: a low-precision
    position collapses nearby positions, so the angle is formed in float64).
    dtype "f64" keeps the exact rotation, for derivative checks."""
    if dtype == "f64":
        return rope_rotate(x, pos, base)
    return round_to_dtype(rope_rotate(x, pos, base), dtype)


def _allowed(B, Tq, Tkv, q_pos, kv_pos, causal, kpm, attn_mask, window=(-1, -1)) -> np.ndarray:
    """allowed[b, i, j]: key-padding and attention-mask exclusions combined
    ("Transformers and Attention" #2), if causal, key position <= query
    position (#24), and the sliding window: a key at most `left` positions
    before and at most `right` positions after the query (#55, Longformer:
    each token connects to nearby positions; the post's flash-attention call
    passes the window as a (left, right) pair, -1 meaning no limit on that
    side)."""
    allowed = np.ones((B, Tq, Tkv), dtype=bool)
    if kpm is not None:
        allowed &= ~(np.asarray(kpm) != 0)[:, None, :]
    if attn_mask is not None:
        allowed &= ~(np.asarray(attn_mask) != 0)[None, :, :]
    qp = np.asarray(q_pos)[None, :, None]
    kp = np.asarray(kv_pos)[None, None, :]
    if causal:
        allowed &= kp <= qp
    left, right = window
    if left >= 0:
        allowed &= kp >= qp - left
    if right >= 0:
        allowed &= kp <= qp + right
    return allowed


def alibi_bias(q_pos, kv_pos, slope: float) -> np.ndarray:
    """ALiBi ("Transformers and Attention" #58): a penalty proportional to the
    query-key distance, with a fixed slope per head, added to the scores
    before the softmax: -slope * |pos_q - pos_k|, shape (Tq, Tkv).  It is
    added to the scaled scores (the scores softmax sees); the absolute
    distance makes it symmetric when keys lie after the query."""
    qp = np.asarray(q_pos, dtype=np.float64)[:, None]
    kp = np.asarray(kv_pos, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(qp - kp)


def sdpa(q, k, v, q_pos, kv_pos, *, causal: bool = False, kpm=None, attn_mask=None,
         rope_base: float = 0.0, dtype: str = "bf16", window=(-1, -1),
         alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """out, lse of softmax(q k^T / sqrt(d) + mask) v for every (batch, head).

    q: (B, Tq, H, d), k and v: (B, Tkv, H, d) holding the exact input values;
    q_pos[Tq], kv_pos[Tkv]: absolute token positions (causal test and RoPE).
    kpm: (B, Tkv), nonzero = ignored key; attn_mask: (Tq, Tkv), nonzero =
    forbidden pair.  Their exclusions combine ("Transformers and Attention"
    #2), and causal order keeps the diagonal and everything before it (#24;
    "CP: Split Long Contexts Across GPUs", "Why attention needs information
    from other GPUs": t3 attends to t0..t3).

    With rope_base > 0, q and k are first rotated in float64 and rounded
    once to ``dtype`` (``_rotated``), as if the rotation had been applied to
    the stored tensors.  Scores are scaled by 1/sqrt(d) (#15, #22).  Row softmax is the two-pass
    safe form (brunomaga.github.io post, "Improving numerical stability"):
    m = max of the allowed scores, e = exp(s - m) on allowed entries and
    exactly 0 elsewhere, l = sum e, out = (e / l) v, lse = m + ln l (the
    log-sum-exp of the allowed scores, "LSE" in the same section).
    A row with no allowed key returns out = 0 and lse = -inf.
    window = (left, right) limits the keys to a band around each query
    (``_allowed``); alibi_slopes[H], if given, adds ``alibi_bias`` with the
    head's slope to the scaled scores (lse then includes the bias).

    Returns out (B, Tq, H, d_v) and lse (B, H, Tq), both float64 (the value
    width d_v may differ from d, "Transformers and Attention" #24).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Tq, H, d = q.shape
    Tkv = k.shape[1]
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    if rope_base > 0:
        q = _rotated(q, q_pos, rope_base, dtype)
        k = _rotated(k, kv_pos, rope_base, dtype)
    allowed = _allowed(B, Tq, Tkv, q_pos, kv_pos, causal, kpm, attn_mask, window)

    scale = 1.0 / math.sqrt(d)
    dv = v.shape[-1]
    out = np.zeros((B, Tq, H, dv), dtype=np.float64)
    lse = np.full((B, H, Tq), NEG_INF, dtype=np.float64)
    for b in range(B):
        ok = allowed[b]
        has = ok.any(axis=1)
        for h in range(H):
            s = scale * (q[b, :, h, :] @ k[b, :, h, :].T)            # (Tq, Tkv)
            if alibi_slopes is not None:
                s = s + alibi_bias(q_pos, kv_pos, alibi_slopes[h])
            sm = np.where(ok, s, NEG_INF)
            m = np.max(sm, axis=1) if Tkv else np.full(Tq, NEG_INF)
            m_safe = np.where(has, m, 0.0)
            with np.errstate(over="ignore"):                        # masked garbage may overflow; it is discarded
                e = np.where(ok, np.exp(s - m_safe[:, None]), 0.0)
            l = e.sum(axis=1)
            l_safe = np.where(has, l, 1.0)
            p = e / l_safe[:, None]
            out[b, :, h, :] = p @ v[b, :, h, :]
            lse[b, h, :] = np.where(has, m_safe + np.log(l_safe), NEG_INF)
    return out, lse


def sdpa_backward(q, k, v, dout, q_pos, kv_pos, *, causal: bool = False, kpm=None, attn_mask=None,
                  rope_base: float = 0.0, dtype: str = "bf16", window=(-1, -1),
                  alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients dq, dk, dv of L = sum_i dout_i . out_i for the ``sdpa``
    forward with the same arguments.

    The brunomaga.github.io post ("Ring Attention", item 3; "Implementation",
    the backward pass) states that the backward pass is computed blockwise
    from dout, q, k, v, the final out and the saved log-sum-exp, with dq
    accumulated locally and dk, dv accumulated alongside their K/V block.  The
    block gradients are those of the whole attention, so the plain definition
    is the chain rule through the forward definition, written out here with
    the full probability matrix:
        P = softmax of the allowed scores (exactly 0 elsewhere),
        dv_j  = sum_i P_ij dout_i,
        dP_ij = dout_i . v_j,
        dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
        dq'_i = (1/sqrt(d)) sum_j dS_ij k'_j,   dk'_j = (1/sqrt(d)) sum_i dS_ij q'_i,
    and with RoPE dq = R(pos)^T dq', dk = R(pos)^T dk' (the rotation is
    orthogonal).  The rounding of the rotated operands to the input dtype is
    passed through unchanged (its derivative is taken as the identity).
    A row with no allowed key contributes nothing.  A window removes pairs
    like a mask; an ALiBi penalty enters P only (it does not depend on q or
    k), so both carry over from ``sdpa`` unchanged.

    Shapes as in ``sdpa``; dout is (B, Tq, H, d_v).  Returns float64 dq
    (B, Tq, H, d), dk (B, Tkv, H, d), dv (B, Tkv, H, d_v).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Tq, H, d = q.shape
    Tkv = k.shape[1]
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    qr, kr = q, k
    if rope_base > 0:
        qr = _rotated(q, q_pos, rope_base, dtype)
        kr = _rotated(k, kv_pos, rope_base, dtype)
    allowed = _allowed(B, Tq, Tkv, q_pos, kv_pos, causal, kpm, attn_mask, window)
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(qr)
    dk = np.zeros_like(kr)
    dv = np.zeros_like(v)
    for b in range(B):
        ok = allowed[b]
        has = ok.any(axis=1)
        for h in range(H):
            s = scale * (qr[b, :, h, :] @ kr[b, :, h, :].T)
            if alibi_slopes is not None:
                s = s + alibi_bias(q_pos, kv_pos, alibi_slopes[h])
            m = np.where(has, np.max(np.where(ok, s, NEG_INF), axis=1) if Tkv else 0.0, 0.0)
            with np.errstate(over="ignore"):
                e = np.where(ok, np.exp(s - m[:, None]), 0.0)
            l = np.where(has, e.sum(axis=1), 1.0)
            p = e / l[:, None]                                        # (Tq, Tkv)
            g = dout[b, :, h, :]
            dp = g @ v[b, :, h, :].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dv[b, :, h, :] = p.T @ g
            dq[b, :, h, :] = scale * (ds @ kr[b, :, h, :])
            dk[b, :, h, :] = scale * (ds.T @ qr[b, :, h, :])
    if rope_base > 0:
        dq = rope_rotate(dq, -q_pos, rope_base)
        dk = rope_rotate(dk, -kv_pos, rope_base)
    return dq, dk, dv


def key_block_gradients(q, k, v, dout, out, lse, q_pos, kv_pos, key_rows, *, causal: bool = False, kpm=None,
                        rope_base: float = 0.0, dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """dk, dv of the key rows ``key_rows`` alone, from dout, q, k, v and the
    forward's final out and lse of every query row.

    This is the block gradient of the brunomaga.github.io post ("Ring
    Attention", item 3; "Implementation", the backward pass): a K/V block's
    dk, dv follow from dout, the operands, the final out and the saved
    log-sum-exp, without the other keys.  With s_ij the scaled score of the
    rotated q'_i, k'_j and lse_i, out_i those of ``sdpa`` over all keys:
        P_ij  = exp(s_ij - lse_i) on allowed pairs, 0 elsewhere,
        dP_ij = dout_i . v_j,   delta_i = dout_i . out_i (= sum_l P_il dP_il),
        dv_j  = sum_i P_ij dout_i,
        dk'_j = (1/sqrt(d)) sum_i P_ij (dP_ij - delta_i) q'_i,   dk_j = R(pos_j)^T dk'_j,
    the same chain rule as ``sdpa_backward``, restricted to the listed keys
    (rows with lse = -inf see no key and contribute nothing).

    q, dout: (B, Tq, H, d); k, v: (B, Tkv, H, d); out: (B, Tq, H, d) and lse
    (B, H, Tq) from ``sdpa`` with the same arguments; key_rows: indices into
    the key axis.  Returns float64 dk, dv of shape (B, len(key_rows), H, d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    key_rows = np.asarray(key_rows, dtype=np.int64)
    B, Tq, H, d = q.shape
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)[key_rows]
    k = k[:, key_rows]
    v = v[:, key_rows]
    qr, kr = q, k
    if rope_base > 0:
        qr = _rotated(q, q_pos, rope_base, dtype)
        kr = _rotated(k, kv_pos, rope_base, dtype)
    kpm_sel = None if kpm is None else np.asarray(kpm)[:, key_rows]
    allowed = _allowed(B, Tq, len(key_rows), q_pos, kv_pos, causal, kpm_sel, None)
    scale = 1.0 / math.sqrt(d)
    dk = np.zeros_like(kr)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            ls = lse[b, h]
            ok = allowed[b] & np.isfinite(ls)[:, None]
            s = scale * (qr[b, :, h, :] @ kr[b, :, h, :].T)           # (Tq, n keys)
            with np.errstate(over="ignore", invalid="ignore"):
                p = np.where(ok, np.exp(s - np.where(np.isfinite(ls), ls, 0.0)[:, None]), 0.0)
            g = dout[b, :, h, :]
            dp = g @ v[b, :, h, :].T
            delta = (g * out[b, :, h, :]).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dv[b, :, h, :] = p.T @ g
            dk[b, :, h, :] = scale * (ds.T @ qr[b, :, h, :])
    if rope_base > 0:
        dk = rope_rotate(dk, -kv_pos, rope_base)
    return dk, dv


def attention_backward(q, k, v, dout, *, q_off: int = 0, kv_off: int = 0, **kw):
    """``sdpa_backward`` with contiguous positions q_off + i and kv_off + j."""
    Tq = np.asarray(q).shape[1]
    Tkv = np.asarray(k).shape[1]
    return sdpa_backward(q, k, v, dout, q_off + np.arange(Tq), kv_off + np.arange(Tkv), **kw)


def attention(q, k, v, *, q_off: int = 0, kv_off: int = 0, **kw) -> Tuple[np.ndarray, np.ndarray]:
    """``sdpa`` with contiguous positions q_off + i and kv_off + j."""
    Tq = np.asarray(q).shape[1]
    Tkv = np.asarray(k).shape[1]
    return sdpa(q, k, v, q_off + np.arange(Tq), kv_off + np.arange(Tkv), **kw)


# --------------------------------------------------------------------------
# decoding over a key/value cache
# --------------------------------------------------------------------------
def kv_append(k_cache, v_cache, cache_len, k_new, v_new, *, rope_base: float = 0.0,
              dtype: str = "bf16"):
    """One decoding step's cache update ("Transformers and Attention" #53: the
    new token's key and value are appended to the layer's cache; #57: a
    static cache has a fixed number of slots and masks the unused ones).

    k_cache, v_cache: (B, Tcap, H, d); cache_len[B]: filled slots (slot j
    holds the token at position j); k_new, v_new: (B, H, d).  The new key is
    stored rotated to its position cache_len[b] (``_rotated``: the float64
    rotation rounded once to ``dtype``), the value as given; cache_len[b] grows by
    one.  A full cache (cache_len[b] == Tcap) is left unchanged.  Returns new
    arrays (k_cache, v_cache, cache_len).
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    ln = np.array(cache_len, dtype=np.int64, copy=True)
    Tcap = kc.shape[1]
    for b in range(kc.shape[0]):
        L = int(ln[b])
        if L >= Tcap:
            continue
        kb = np.asarray(k_new[b], dtype=np.float64)[None, :, :]      # (1, H, d)
        if rope_base > 0:
            kb = _rotated(kb, np.array([L]), rope_base, dtype)
        kc[b, L] = kb[0]
        vc[b, L] = np.asarray(v_new[b], dtype=np.float64)
        ln[b] = L + 1
    return kc, vc, ln


def decode(q, k_cache, v_cache, cache_len, *, rope_base: float = 0.0, dtype: str = "bf16",
           window_left: int = -1, alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the newest token over the cache ("Transformers and
    Attention" #53: at step t the new query attends over the retained and
    the current keys and values).

    q: (B, H, d), the query of the token at position cache_len[b] - 1 (its
    key and value already appended); keys are the cache slots [0,
    cache_len[b]) as stored (already rotated by ``kv_append``), the query is
    rotated to its position here.  window_left >= 0 keeps only the keys at
    most that many positions back (#57: windowed layers retain a bounded
    history); alibi_slopes as in ``sdpa``.  Causal order holds by
    construction (no slot after the query is filled).  Returns out (B, H, d)
    and lse (B, H); an empty cache row gives (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, H, d = q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, H, vc.shape[-1]), dtype=np.float64)
    lse = np.full((B, H), NEG_INF, dtype=np.float64)
    for b in range(B):
        L = int(cache_len[b])
        if L <= 0:
            continue
        pos = L - 1
        lo = 0 if window_left < 0 else max(0, pos - window_left)
        qb = q[b][None, :, :]                                        # (1, H, d)
        if rope_base > 0:
            qb = _rotated(qb, np.array([pos]), rope_base, dtype)
        for h in range(H):
            s = scale * (kc[b, lo:L, h, :] @ qb[0, h, :])            # (L - lo,)
            if alibi_slopes is not None:
                s = s + alibi_bias([pos], np.arange(lo, L), alibi_slopes[h])[0]
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            out[b, h, :] = (e / l) @ vc[b, lo:L, h, :]
            lse[b, h] = m + math.log(l)
    return out, lse


# --------------------------------------------------------------------------
# merge of partial (out, lse) results
# --------------------------------------------------------------------------
def merge(out_a, lse_a, out_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Combine two partial results over disjoint key sets.

    The pages call an accumulate function for each ring step but never define
    it; this follows from the fraction form of attention (brunomaga.github.io
    post, "Ring Attention": out = sum exp(s) v / sum exp(s)), the rescale of
    both accumulators by exp of the max difference and the LogSumExp carry
    ("Improving numerical stability"), and the warning that block outputs must
    not simply be added or averaged ("CP: Split Long Contexts Across GPUs",
    "Circulate K/V blocks with Ring").

    lse = m* + ln(e^(lse_a - m*) + e^(lse_b - m*)), m* = max(lse_a, lse_b);
    out = e^(lse_a - lse) out_a + e^(lse_b - lse) out_b.  (0, -inf) is the
    identity; two empty partials give (0, -inf).
    out_*: (B, Tq, H, d); lse_*: (B, H, Tq).
    """
    oa = np.asarray(out_a, dtype=np.float64)
    ob = np.asarray(out_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    mx = np.maximum(la, lb)
    empty = ~np.isfinite(mx)
    mx_safe = np.where(empty, 0.0, mx)
    with np.errstate(invalid="ignore"):
        tot = np.exp(la - mx_safe) + np.exp(lb - mx_safe)
    lse = np.where(empty, NEG_INF, mx_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    wa = np.where(empty, 0.0, np.exp(la - lse_safe))                  # (B, H, Tq)
    wb = np.where(empty, 0.0, np.exp(lb - lse_safe))
    wa = np.transpose(wa, (0, 2, 1))[..., None]                      # (B, Tq, H, 1)
    wb = np.transpose(wb, (0, 2, 1))[..., None]
    out = wa * oa + wb * ob
    return out, lse


# --------------------------------------------------------------------------
# ring placement and order (integer bookkeeping)
# --------------------------------------------------------------------------
def ring_order(P: int, rank: int) -> List[int]:
    """Blocks rank ``rank`` sees, in order: its own, then the one of the
    previous rank, and so on ("CP: Split Long Contexts Across GPUs", "Circulate
    K/V blocks with Ring": GPU 0 of 4 sees K0, K3, K2, K1; brunomaga.github.io
    post, "Distributed algorithm": P steps, receive from the previous rank)."""
    return [(rank - s) % P for s in range(P)]


def zigzag_chunks(P: int, rank: int) -> Tuple[int, int]:
    """Chunks of size T/(2P) owned by ``rank`` under the load-balanced causal
    placement: an early chunk and its mirror ("CP: Split Long Contexts Across
    GPUs", "Balance the workload in causal attention": with P = 2 and 8 tokens
    GPU 0 owns t0, t1, t6, t7)."""
    return rank, 2 * P - 1 - rank


def local_query_positions(T: int, P: int, rank: int, zigzag: bool) -> np.ndarray:
    """Absolute positions of the query rows a rank owns (also the positions
    of the K/V block it starts the ring with)."""
    if zigzag:
        c = T // (2 * P)
        a, b = zigzag_chunks(P, rank)
        return np.concatenate([np.arange(a * c, (a + 1) * c), np.arange(b * c, (b + 1) * c)])
    c = T // P
    return np.arange(rank * c, (rank + 1) * c)


def allowed_pairs(q_pos: Iterable[int], kv_pos: Iterable[int], causal: bool = True) -> int:
    """Brute-force count of allowed (query, key) pairs."""
    qp = np.asarray(list(q_pos), dtype=np.int64)
    kp = np.asarray(list(kv_pos), dtype=np.int64)
    if not causal:
        return int(qp.size * kp.size)
    return int((kp[None, :] <= qp[:, None]).sum())


def zigzag_pairs_closed_form(P: int, c: int) -> int:
    """Causal pairs of one zigzag rank with chunk size c: the early chunk r
    sees r*c earlier keys plus its own triangle, the late chunk 2P-1-r sees
    (2P-1-r)*c earlier keys plus its own triangle; the sum is rank-independent,
    (2P-1) c^2 + c (c+1)."""
    return (2 * P - 1) * c * c + c * (c + 1)
