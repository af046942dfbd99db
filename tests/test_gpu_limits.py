"""GPU parity at the size limits of the addressing: key/value tensors past
4 GiB, so every byte offset of a key row beyond the first 2^32 bytes needs
the 64-bit tile bases, with positions near 2^40.

Inputs are drawn on the device from a seeded generator (a few GiB would take
minutes to draw on the host); the oracle sees the exact bf16 values of the
heads it checks, copied back.  The oracle's rotary angles (base^(-2t/d)
times the position) and the library's (exp of -2t/d ln base, times the
position) agree to a few float64 ulps of the frequency; at positions near
2^40 that is about 1e-4 rad, well inside the bf16 tolerances (at 2^52 it
would not be, which is why the positions here stop at 2^40).
"""
import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
from gpu_helpers import DEV, TOL, note, np64

pytestmark = pytest.mark.gpu


def _draw(shape, seed, sigma=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * sigma).to(torch.bfloat16)


def _check(got_o, got_l, ref_o, ref_l, what):
    tol_o, tol_l = TOL["bf16"]
    eo = float(np.abs(got_o - ref_o).max())
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), fin), f"{what}: empty-row pattern differs"
    el = float(np.abs(got_l[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    note(f"  {what}: max|out err| {eo:.3e}  max|lse err| {el:.3e}")
    assert eo <= tol_o and el <= tol_l, what


def test_forward_keys_past_4gib():
    """2^18 + 1000 keys x 64 heads x d = 128 in bf16: k and v are just over
    4 GiB each (key row stride 16 KiB, so the last 1000 keys start past byte
    2^32), causal with the queries at positions 2^40 .. 2^40 + 299 and the
    keys ending 150 positions after the first query, a random key-padding
    mask plus a padded tail, RoPE base 10000.  Sampled query rows of the
    first and the last head against the oracle over all keys."""
    B, H, d = 1, 64, 128
    Tkv, Tq = (1 << 18) + 1000, 300
    assert (Tkv - 1) * H * d * 2 >= 1 << 32
    q_off = 1 << 40
    kv_off = q_off - Tkv + 150
    note(f"limits forward: B={B} H={H} Tq={Tq} Tkv={Tkv} d={d} q_off=2^40 kv_off=q_off-{Tkv - 150}")
    q = _draw((B, Tq, H, d), 71)
    k = _draw((B, Tkv, H, d), 72)
    v = _draw((B, Tkv, H, d), 73)
    g = torch.Generator(device=DEV)
    g.manual_seed(74)
    kpm = (torch.rand((B, Tkv), generator=g, device=DEV) < 0.1).to(torch.uint8)
    kpm[:, Tkv - 20:] = 1
    out, lse = bosa.attn_fwd(q, k, v, q_off=q_off, kv_off=kv_off, causal=True, kpm=kpm, rope_base=10000.0)
    torch.cuda.synchronize()
    sel = np.r_[0:24, 140:160, 276:300]          # both query tiles, the causal edge, the ragged end
    kpm_h = kpm.cpu().numpy()
    kv_pos = kv_off + np.arange(Tkv, dtype=np.int64)
    for h in (0, H - 1):
        ro, rl = oracle.sdpa(np64(q[:, sel, h:h + 1]), np64(k[:, :, h:h + 1]), np64(v[:, :, h:h + 1]),
                             q_off + sel.astype(np.int64), kv_pos, causal=True, kpm=kpm_h, rope_base=10000.0,
                             dtype="bf16")
        _check(np64(out[:, sel, h:h + 1]), np64(lse[:, h:h + 1, sel]), ro, rl, f"head {h}")


def test_decode_cache_past_4gib():
    """A static cache of 2^20 + 100 slots x 16 heads x d = 128 for each of
    2 rows (4 GiB per row, 8 GiB per tensor) filled to 2^20 + 77 and 300000
    slots: append one token per row, then decode its query; two heads
    against the oracle."""
    B, H, d = 2, 16, 128
    Tcap = (1 << 20) + 100
    note(f"limits decode: B={B} H={H} Tcap={Tcap} d={d}")
    kc = _draw((B, Tcap, H, d), 81)
    vc = _draw((B, Tcap, H, d), 82)
    ln = torch.tensor([(1 << 20) + 77, 300000], dtype=torch.int32, device=DEV)
    kn, vn, qn = _draw((B, H, d), 83), _draw((B, H, d), 84), _draw((B, H, d), 85)
    bosa.attn_kv_append(kn, vn, kc, vc, ln, rope_base=10000.0)
    out, lse = bosa.attn_decode(qn, kc, vc, ln, rope_base=10000.0)
    torch.cuda.synchronize()
    lh = ln.cpu().numpy()
    assert lh.tolist() == [(1 << 20) + 78, 300001]
    for h in (3, 15):
        ro, rl = oracle.decode(np64(qn[:, h:h + 1]), np64(kc[:, :, h:h + 1]), np64(vc[:, :, h:h + 1]), lh,
                               rope_base=10000.0, dtype="bf16")
        _check(np64(out[:, h:h + 1]), np64(lse[:, h:h + 1]), ro, rl, f"head {h}")


def test_backward_keys_past_4gib():
    """The backward of the forward case above (2^18 + 1000 keys x 64 heads,
    k and v just over 4 GiB, causal, key padding, RoPE at positions near
    2^40): dq, dk and dv of the last head, whose rows reach furthest into
    each key row, against the backward oracle, to the tolerance of the other
    backward tests (largest error relative to the tensor's largest value)."""
    from test_gpu_backward import compare_grads

    B, H, d = 1, 64, 128
    Tkv, Tq = (1 << 18) + 1000, 300
    q_off = 1 << 40
    kv_off = q_off - Tkv + 150
    note(f"limits backward: B={B} H={H} Tq={Tq} Tkv={Tkv} d={d} q_off=2^40 kv_off=q_off-{Tkv - 150}")
    q = _draw((B, Tq, H, d), 91)
    k = _draw((B, Tkv, H, d), 92)
    v = _draw((B, Tkv, H, d), 93)
    dout = _draw((B, Tq, H, d), 94)
    g = torch.Generator(device=DEV)
    g.manual_seed(95)
    kpm = (torch.rand((B, Tkv), generator=g, device=DEV) < 0.1).to(torch.uint8)
    kpm[:, Tkv - 20:] = 1
    kw = dict(q_off=q_off, kv_off=kv_off, causal=True, kpm=kpm, rope_base=10000.0)
    out, lse = bosa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = bosa.attn_bwd(q, k, v, out, dout, lse, **kw)
    torch.cuda.synchronize()
    h = H - 1
    ref = oracle.attention_backward(np64(q[:, :, h:h + 1]), np64(k[:, :, h:h + 1]), np64(v[:, :, h:h + 1]),
                                    np64(dout[:, :, h:h + 1]), q_off=q_off, kv_off=kv_off, causal=True,
                                    kpm=kpm.cpu().numpy(), rope_base=10000.0, dtype="bf16")
    compare_grads([x[:, :, h:h + 1].cpu() for x in (dq, dk, dv)], ref, f"head {h}")
