"""Seeded random sweep of the GPU path against the oracle.

Each case draws its shape, positions, masks, rotary base, window and ALiBi
slopes from its own generator (seed = a fixed base + the case number), so a
failure names a case that replays exactly.  Sizes stay small enough for the
oracle; they are ragged on purpose (neither rows nor keys a multiple of the
64-key tile or the 32-row wave).  Forward in both dtypes, backward, ring
shares and decoding; the tolerances are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
import workloads
from gpu_helpers import DEV, chained_ring_reference, compare, note, np64
from test_gpu_backward import compare_grads

pytestmark = pytest.mark.gpu

N_FWD, N_BWD, N_RING, N_DEC = 200, 60, 40, 40
N_BWD_BF16 = 40
# cases of a longer sweep that sit at the edges of the float32 tolerances:
# forward with ALiBi at distances near 1000 (|lse| in the hundreds), backward
# with rows that see a single key (exact gradients cancel to zero)
EXTRA_FWD, EXTRA_BWD = [2152, 2310], [426, 571]


def _draw(shape, seed, dtype):
    return workloads.random_normal(shape, seed, dtype)


def _variant(rng, H, span):
    """A window (30% of cases) with each side either unlimited or up to
    `span` positions, and ALiBi slopes (25% of cases)."""
    window = None
    if rng.random() < 0.3:
        side = lambda: -1 if rng.random() < 0.3 else int(rng.integers(0, span))
        window = (side(), side())
    slopes = workloads.alibi_slopes(H) if rng.random() < 0.25 else None
    return window, slopes


def _mask(shape, seed, p):
    return workloads.random_mask(shape, seed, p) if p > 0 else None


def _oracle_kw(window, slopes):
    return dict(window=(-1, -1) if window is None else window,
                alibi_slopes=None if slopes is None else slopes.double().numpy())


@pytest.mark.parametrize("case", list(range(N_FWD)) + EXTRA_FWD)
def test_random_forward(case):
    rng = np.random.default_rng(20000 + case)
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    d = int(rng.choice([64, 128]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Tq, Tkv = int(rng.integers(1, 600)), int(rng.integers(1, 700))
    causal = bool(rng.random() < 0.6)
    q_off, kv_off = int(rng.integers(0, 1500)), int(rng.integers(0, 1500))
    kpm_p = float(rng.choice([0.0, 0.0, 0.2, 0.7]))
    am_p = float(rng.choice([0.0, 0.0, 0.0, 0.1]))
    rope = float(rng.choice([0.0, 10000.0, 500.0]))
    window, slopes = _variant(rng, H, 400)
    seed = 21000 + 10 * case
    note(f"random forward {case}: {dtype} d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) "
         f"causal={causal} kpm={kpm_p} amask={am_p} rope={rope} window={window} alibi={slopes is not None}")
    q, k, v = _draw((B, Tq, H, d), seed, dtype), _draw((B, Tkv, H, d), seed + 1, dtype), _draw((B, Tkv, H, d), seed + 2, dtype)
    kpm, am = _mask((B, Tkv), seed + 3, kpm_p), _mask((Tq, Tkv), seed + 4, am_p)
    out, lse = bosa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), q_off=q_off, kv_off=kv_off, causal=causal,
                             kpm=None if kpm is None else kpm.to(DEV), attn_mask=None if am is None else am.to(DEV),
                             rope_base=rope, window=window, alibi_slopes=None if slopes is None else slopes.to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(np64(q), np64(k), np64(v), q_off=q_off, kv_off=kv_off, causal=causal,
                              kpm=None if kpm is None else kpm.numpy(), attn_mask=None if am is None else am.numpy(),
                              rope_base=rope, dtype="f32" if dtype == torch.float32 else "bf16",
                              **_oracle_kw(window, slopes))
    compare(out.cpu(), lse.cpu(), ro, rl, "f32" if dtype == torch.float32 else "bf16", f"case {case}")


def _backward_case(case):
    """Inputs and call arguments of random backward case `case`."""
    rng = np.random.default_rng(22000 + case)
    d = int(rng.choice([64, 128]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    Tq, Tkv = int(rng.integers(1, 400)), int(rng.integers(1, 500))
    causal = bool(rng.random() < 0.6)
    q_off, kv_off = int(rng.integers(0, 1000)), int(rng.integers(0, 1000))
    kpm_p = float(rng.choice([0.0, 0.0, 0.3]))
    am_p = float(rng.choice([0.0, 0.0, 0.0, 0.1]))
    rope = float(rng.choice([0.0, 10000.0]))
    window, slopes = _variant(rng, H, 300)
    seed = 23000 + 10 * case
    note(f"random backward {case}: d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) causal={causal} "
         f"kpm={kpm_p} amask={am_p} rope={rope} window={window} alibi={slopes is not None}")
    bf = torch.bfloat16
    q, k, v = _draw((B, Tq, H, d), seed, bf), _draw((B, Tkv, H, d), seed + 1, bf), _draw((B, Tkv, H, d), seed + 2, bf)
    dout = _draw((B, Tq, H, d), seed + 3, bf)
    kpm, am = _mask((B, Tkv), seed + 4, kpm_p), _mask((Tq, Tkv), seed + 5, am_p)
    kw = dict(q_off=q_off, kv_off=kv_off, causal=causal, kpm=None if kpm is None else kpm.to(DEV),
              attn_mask=None if am is None else am.to(DEV), rope_base=rope, window=window,
              alibi_slopes=None if slopes is None else slopes.to(DEV))
    return (q, k, v, dout, kpm, am), kw, (q_off, kv_off, causal, rope, window, slopes)


@pytest.mark.parametrize("case", list(range(N_BWD)) + EXTRA_BWD)
def test_random_backward(case):
    (q, k, v, dout, kpm, am), kw, (q_off, kv_off, causal, rope, window, slopes) = _backward_case(case)
    qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    out, lse = bosa.attn_fwd(qd, kd, vd, **kw)
    grads = bosa.attn_bwd(qd, kd, vd, out, od, lse, flags=bosa.ATTN_OUT_F32, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(dout), q_off=q_off, kv_off=kv_off,
                                    causal=causal, kpm=None if kpm is None else kpm.numpy(),
                                    attn_mask=None if am is None else am.numpy(), rope_base=rope, dtype="bf16",
                                    **_oracle_kw(window, slopes))
    compare_grads([g.cpu() for g in grads], ref, f"case {case}")


@pytest.mark.parametrize("case", range(N_BWD_BF16))
def test_random_backward_bf16_gradients_equal_rounded_float32(case):
    """The bf16 gradients of a call (dk and dv written as final bf16 by the
    dK/dV kernel, dk rotated back first; dq through the finalize pass) equal
    the float32 gradients of the same call rounded to bf16: bit for bit for
    dv, and for dk and dq without RoPE.  With RoPE the bf16 path rounds the
    float64 back-rotation once, the float32 path rounds it to float32 and then
    to bf16, which can differ by one bf16 unit where the float32 value lands
    on a bf16 midpoint."""
    (q, k, v, dout, _, _), kw, (_, _, _, rope, _, _) = _backward_case(1000 + case)
    qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    out, lse = bosa.attn_fwd(qd, kd, vd, **kw)
    g16 = bosa.attn_bwd(qd, kd, vd, out, od, lse, **kw)
    g32 = bosa.attn_bwd(qd, kd, vd, out, od, lse, flags=bosa.ATTN_OUT_F32, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g16, g32):
        assert a.dtype == torch.bfloat16 and b.dtype == torch.float32, name
        ia = a.cpu().view(torch.int16).to(torch.int32)
        ib = b.cpu().to(torch.bfloat16).view(torch.int16).to(torch.int32)
        if rope > 0 and name != "dv":
            # one unit apart at most (same sign: the bit patterns are adjacent)
            diff = (ia - ib).abs()
            n = int((diff != 0).sum())
            assert int(diff.max()) <= 1 if diff.numel() else True, f"case {case} {name}: more than one bf16 unit"
            assert n <= max(2, diff.numel() // 1000), f"case {case} {name}: {n} of {diff.numel()} differ"
        else:
            assert torch.equal(ia, ib), f"case {case} {name}: not bit-identical"


@pytest.mark.parametrize("case", range(N_RING))
def test_random_ring_share(case):
    rng = np.random.default_rng(24000 + case)
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    d = int(rng.choice([64, 128]))
    P = int(rng.choice([2, 4]))
    zigzag = bool(rng.random() < 0.5)
    c = int(rng.integers(20, 160))
    T = (2 * P if zigzag else P) * c
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal = bool(rng.random() < 0.7)
    rank = int(rng.integers(0, P))
    kpm_p = float(rng.choice([0.0, 0.2]))
    rope = float(rng.choice([0.0, 10000.0]))
    window, slopes = _variant(rng, H, 2 * c)
    seed = 25000 + 10 * case
    note(f"random ring {case}: {dtype} d={d} P={P} zigzag={zigzag} T={T} B={B} H={H} rank={rank} causal={causal} "
         f"kpm={kpm_p} rope={rope} window={window} alibi={slopes is not None}")
    q = _draw((B, T // P, H, d), seed, dtype)
    k, v = _draw((B, T, H, d), seed + 1, dtype), _draw((B, T, H, d), seed + 2, dtype)
    kpm = _mask((B, T), seed + 3, kpm_p)
    out, lse = bosa.attn_ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P=P, rank=rank, zigzag=zigzag, causal=causal,
                                  kpm=None if kpm is None else kpm.to(DEV), rope_base=rope, window=window,
                                  alibi_slopes=None if slopes is None else slopes.to(DEV))
    torch.cuda.synchronize()
    qpos = oracle.local_query_positions(T, P, rank, zigzag)
    ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=causal,
                         kpm=None if kpm is None else kpm.numpy(), rope_base=rope,
                         dtype="f32" if dtype == torch.float32 else "bf16", **_oracle_kw(window, slopes))
    compare(out.cpu(), lse.cpu(), ro, rl, "f32" if dtype == torch.float32 else "bf16", f"case {case}")


@pytest.mark.parametrize("case", range(N_DEC))
def test_random_decode(case):
    rng = np.random.default_rng(26000 + case)
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    d = int(rng.choice([64, 128]))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    Tcap = int(rng.integers(1, 3000))
    lens = rng.integers(0, Tcap + 1, size=B)
    rope = float(rng.choice([0.0, 10000.0]))
    wl = -1 if rng.random() < 0.6 else int(rng.integers(0, 500))
    slopes = workloads.alibi_slopes(H) if rng.random() < 0.3 else None
    seed = 27000 + 10 * case
    note(f"random decode {case}: {dtype} d={d} B={B} H={H} Tcap={Tcap} lens={lens.tolist()} rope={rope} "
         f"window_left={wl} alibi={slopes is not None}")
    kc, vc = _draw((B, Tcap, H, d), seed, dtype), _draw((B, Tcap, H, d), seed + 1, dtype)
    qn = _draw((B, H, d), seed + 2, dtype)
    ln = torch.tensor(lens, dtype=torch.int32)
    out, lse = bosa.attn_decode(qn.to(DEV), kc.to(DEV), vc.to(DEV), ln.to(DEV), rope_base=rope, window_left=wl,
                                alibi_slopes=None if slopes is None else slopes.to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.decode(np64(qn), np64(kc), np64(vc), lens, rope_base=rope,
                           dtype="f32" if dtype == torch.float32 else "bf16", window_left=wl,
                           alibi_slopes=None if slopes is None else slopes.double().numpy())
    compare(out.cpu(), lse.cpu(), ro, rl, "f32" if dtype == torch.float32 else "bf16", f"case {case}")


N_CHAIN = 40


@pytest.mark.parametrize("case", range(N_CHAIN))
def test_random_ring_share_bitwise_against_its_subcalls(case):
    """attn_ring_fwd (bf16: sub-calls chained up to sixteen to a launch, the
    softmax state carried across them) against one attn_fwd call per launch
    over that launch's keys in ring order (causal order as an attention mask,
    rotations applied beforehand), merging into a float32 accumulator, then
    the cast: out and lse bit for bit, over random P (2, 3, 4, 8), layouts,
    head counts, key padding and ranks."""
    rng = np.random.default_rng(50000 + case)
    P = int(rng.choice([2, 3, 4, 8]))
    zigzag = bool(rng.random() < 0.5)
    c = int(rng.integers(8, 300))
    T = (2 * P if zigzag else P) * c
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    rank = int(rng.integers(0, P))
    rope = float(rng.choice([0.0, 10000.0]))
    kp = float(rng.choice([0.0, 0.0, 0.3]))
    note(f"random ring bitwise {case}: P={P} zigzag={zigzag} T={T} B={B} H={H} d={d} causal={causal} "
         f"rank={rank} rope={rope} kpm={kp}")
    bf = torch.bfloat16
    q = _draw((B, T // P, H, d), 60000 + case, bf).to(DEV)
    k = _draw((B, T, H, d), 61000 + case, bf).to(DEV)
    v = _draw((B, T, H, d), 62000 + case, bf).to(DEV)
    kpm = None
    if kp > 0:
        kpm = workloads.random_mask((B, T), 63000 + case, kp)
        if rng.random() < 0.5:
            kpm[int(rng.integers(0, B)), int(rng.integers(0, T)):] = 1
        kpm = kpm.to(DEV)
    out, lse = bosa.attn_ring_fwd(q, k, v, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=kpm, rope_base=rope)
    ro, rl = chained_ring_reference(q, k, v, kpm, P, rank, zigzag, causal, rope)
    assert torch.equal(out.view(torch.int16), ro.view(torch.int16)), "out differs from the chained launches'"
    assert torch.equal(lse, rl), "lse differs from the chained launches'"


N_RING_BWD = 20


@pytest.mark.parametrize("case", range(N_RING_BWD))
def test_random_ring_backward(case):
    """attn_ring_bwd over random P (2, 3, 4, 8), layouts, head counts, key
    padding and ranks (the first sub-call to touch a block's gradients writes
    them, later ones add, untouched rows are zeroed) against the backward
    oracle over the local rows and every key."""
    rng = np.random.default_rng(80000 + case)
    P = int(rng.choice([2, 3, 4, 8]))
    zigzag = bool(rng.random() < 0.5)
    c = int(rng.integers(8, 200))
    T = (2 * P if zigzag else P) * c
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    rank = int(rng.integers(0, P))
    rope = float(rng.choice([0.0, 10000.0]))
    kp = float(rng.choice([0.0, 0.0, 0.3]))
    note(f"random ring backward {case}: P={P} zigzag={zigzag} T={T} B={B} H={H} d={d} causal={causal} rank={rank} "
         f"rope={rope} kpm={kp}")
    bf = torch.bfloat16
    q, dout = _draw((B, T // P, H, d), 81000 + case, bf), _draw((B, T // P, H, d), 84000 + case, bf)
    k, v = _draw((B, T, H, d), 82000 + case, bf), _draw((B, T, H, d), 83000 + case, bf)
    kpm = _mask((B, T), 85000 + case, kp)
    qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    md = None if kpm is None else kpm.to(DEV)
    out, lse = bosa.attn_ring_fwd(qd, kd, vd, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=md, rope_base=rope)
    grads = bosa.attn_ring_bwd(qd, kd, vd, out, od, lse, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=md,
                               rope_base=rope)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(np64(q), np64(k), np64(v), np64(dout), oracle.local_query_positions(T, P, rank, zigzag),
                               np.arange(T), causal=causal, kpm=None if kpm is None else kpm.numpy(), rope_base=rope,
                               dtype="bf16")
    compare_grads([g.cpu() for g in grads], ref, f"case {case}")
