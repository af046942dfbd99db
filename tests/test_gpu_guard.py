"""Out-of-bounds write checks (GPU).

Every output a call writes lives inside a larger device buffer whose bytes
before and after it hold a sentinel pattern; after the call the sentinel must
be intact, and the inputs must be bit-identical to what was passed.  Shapes are
ragged on purpose: query and key counts that are not multiples of 32, 64 or
256, and B * H not a multiple of 8, so the kernels' tails, partial tiles and
grid remainders all run.  The checks read only memory the test owns, so a
stray write shows up as a changed sentinel byte, never as a fault.
"""
from __future__ import annotations

import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import workloads
from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side (a multiple of 256 keeps the view's alignment)
SENTINEL = 0xA5


class Guarded:
    """A device tensor of `shape`/`dtype` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype, fill=None):
        n = 1
        for s in shape:
            n *= s
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what: str) -> None:
        torch.cuda.synchronize()
        lo = self.raw[:GUARD].cpu()
        hi = self.raw[GUARD + self.nbytes:].cpu()
        bad_lo = int((lo != SENTINEL).sum())
        bad_hi = int((hi != SENTINEL).sum())
        assert bad_lo == 0 and bad_hi == 0, f"{what}: {bad_lo} bytes before and {bad_hi} after the tensor changed"


def rnd(shape, seed, dtype):
    return workloads.random_normal(shape, seed, dtype).to(DEV)


def inputs_unchanged(pairs, what):
    torch.cuda.synchronize()
    for name, (x, x0) in pairs.items():
        assert torch.equal(x.cpu(), x0.cpu()), f"{what}: input {name} was modified"


@pytest.mark.parametrize("dtype,d,B,H,Tq,Tkv,rope,causal", [
    (torch.bfloat16, 128, 3, 3, 333, 517, 10000.0, True),
    (torch.bfloat16, 64, 1, 5, 257, 65, 0.0, False),
    (torch.float32, 64, 1, 5, 77, 130, 10000.0, True),
    (torch.float32, 128, 2, 1, 31, 33, 0.0, False),
])
def test_forward_writes_stay_in_bounds(dtype, d, B, H, Tq, Tkv, rope, causal):
    q, k, v = rnd((B, Tq, H, d), 501, dtype), rnd((B, Tkv, H, d), 502, dtype), rnd((B, Tkv, H, d), 503, dtype)
    kpm = workloads.random_mask((B, Tkv), 504, 0.15).to(DEV)
    saved = {n: (x, x.clone()) for n, x in dict(q=q, k=k, v=v, kpm=kpm).items()}
    note(f"guard fwd {dtype} d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} rope={rope} causal={causal}")
    out = Guarded((B, Tq, H, d), dtype)
    lse = Guarded((B, H, Tq), torch.float32)
    bosa.attn_fwd(q, k, v, out.t, lse.t, q_off=40, kv_off=0, causal=causal, kpm=kpm, rope_base=rope)
    out.check("out")
    lse.check("lse")
    # float32 partial, then a second call merged into it
    acc = Guarded((B, Tq, H, d), torch.float32)
    lse2 = Guarded((B, H, Tq), torch.float32)
    bosa.attn_fwd(q, k, v, acc.t, lse2.t, q_off=40, causal=causal, kpm=kpm, rope_base=rope,
                  flags=bosa.ATTN_OUT_F32)
    bosa.attn_fwd(q, k, v, acc.t, lse2.t, q_off=40, kv_off=Tkv, causal=False, kpm=kpm, rope_base=rope,
                  flags=bosa.ATTN_OUT_F32 | bosa.ATTN_ACCUMULATE)
    acc.check("accumulated out")
    lse2.check("accumulated lse")
    # window and ALiBi variant
    out3 = Guarded((B, Tq, H, d), dtype)
    lse3 = Guarded((B, H, Tq), torch.float32)
    bosa.attn_fwd(q, k, v, out3.t, lse3.t, q_off=40, causal=causal, kpm=kpm, rope_base=rope, window=(100, 7),
                  alibi_slopes=workloads.alibi_slopes(H).to(DEV))
    out3.check("variant out")
    lse3.check("variant lse")
    inputs_unchanged(saved, "forward")


@pytest.mark.parametrize("P,zigzag,dtype,d", [(3, True, torch.bfloat16, 128), (4, False, torch.bfloat16, 64),
                                              (2, True, torch.float32, 64)])
def test_ring_writes_stay_in_bounds(P, zigzag, dtype, d):
    B, H = 2, 3
    T = (2 * P if zigzag else P) * 97
    Tl = T // P
    q, k, v = rnd((B, Tl, H, d), 511, dtype), rnd((B, T, H, d), 512, dtype), rnd((B, T, H, d), 513, dtype)
    kpm = workloads.random_mask((B, T), 514, 0.1).to(DEV)
    saved = {n: (x, x.clone()) for n, x in dict(q=q, k=k, v=v, kpm=kpm).items()}
    note(f"guard ring fwd P={P} zigzag={zigzag} {dtype} d={d} T={T}")
    for rank in (0, P - 1):
        out = Guarded((B, Tl, H, d), dtype)
        lse = Guarded((B, H, Tl), torch.float32)
        acc = Guarded((B, Tl, H, d), torch.float32)
        bosa.attn_ring_fwd(q, k, v, P=P, rank=rank, zigzag=zigzag, causal=True, kpm=kpm, rope_base=10000.0,
                           out=out.t, lse=lse.t, acc=acc.t)
        out.check(f"rank {rank} out")
        lse.check(f"rank {rank} lse")
        acc.check(f"rank {rank} acc")
    inputs_unchanged(saved, "ring forward")


@pytest.mark.parametrize("f32,rope,d", [(False, 10000.0, 128), (True, 0.0, 64), (True, 10000.0, 128)])
def test_backward_writes_stay_in_bounds(f32, rope, d):
    B, H, Tq, Tkv = 3, 3, 301, 187
    dt = torch.bfloat16
    q, k, v = rnd((B, Tq, H, d), 521, dt), rnd((B, Tkv, H, d), 522, dt), rnd((B, Tkv, H, d), 523, dt)
    dout = rnd((B, Tq, H, d), 524, dt)
    kpm = workloads.random_mask((B, Tkv), 525, 0.1).to(DEV)
    out, lse = bosa.attn_fwd(q, k, v, q_off=Tkv - Tq + 50, causal=True, kpm=kpm, rope_base=rope)
    saved = {n: (x, x.clone()) for n, x in dict(q=q, k=k, v=v, dout=dout, out=out, lse=lse).items()}
    gdt = torch.float32 if f32 else dt
    flags = bosa.ATTN_OUT_F32 if f32 else 0
    note(f"guard bwd f32={f32} rope={rope} d={d}")
    dq = Guarded((B, Tq, H, d), gdt)
    dk = Guarded((B, Tkv, H, d), gdt)
    dv = Guarded((B, Tkv, H, d), gdt)
    bosa.attn_bwd(q, k, v, out, dout, lse, dq.t, dk.t, dv.t, q_off=Tkv - Tq + 50, causal=True, kpm=kpm,
                  rope_base=rope, flags=flags)
    if f32:
        bosa.attn_bwd(q, k, v, out, dout, lse, dq.t, dk.t, dv.t, q_off=Tkv - Tq + 50, causal=True, kpm=kpm,
                      rope_base=rope, flags=flags | bosa.ATTN_ACCUMULATE)
    for name, g in dict(dq=dq, dk=dk, dv=dv).items():
        g.check(name)
    inputs_unchanged(saved, "backward")


def test_ring_backward_writes_stay_in_bounds():
    P, B, H, d = 2, 2, 3, 128
    T = 2 * P * 75
    Tl = T // P
    dt = torch.bfloat16
    q, k, v = rnd((B, Tl, H, d), 531, dt), rnd((B, T, H, d), 532, dt), rnd((B, T, H, d), 533, dt)
    dout = rnd((B, Tl, H, d), 534, dt)
    for rank in range(P):
        out, lse = bosa.attn_ring_fwd(q, k, v, P=P, rank=rank, zigzag=True, causal=True, rope_base=10000.0)
        note(f"guard ring bwd rank {rank}")
        dq = Guarded((B, Tl, H, d), dt)
        dk = Guarded((B, T, H, d), dt)
        dv = Guarded((B, T, H, d), dt)
        bosa.attn_ring_bwd(q, k, v, out, dout, lse, P=P, rank=rank, zigzag=True, causal=True, rope_base=10000.0,
                           dq=dq.t, dk=dk.t, dv=dv.t)
        for name, g in dict(dq=dq, dk=dk, dv=dv).items():
            g.check(f"rank {rank} {name}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_decode_writes_stay_in_bounds(dtype, d):
    """attn_kv_append writes slot cache_len[b] of each row with room and
    nothing else of the caches; attn_decode writes out and lse only."""
    B, H, Tcap = 3, 5, 777
    kc = Guarded((B, Tcap, H, d), dtype, rnd((B, Tcap, H, d), 541, dtype))
    vc = Guarded((B, Tcap, H, d), dtype, rnd((B, Tcap, H, d), 542, dtype))
    ln = torch.tensor([0, 400, Tcap], dtype=torch.int32, device=DEV)   # empty, middle, full
    kn, vn, qn = (rnd((B, H, d), 543 + i, dtype) for i in range(3))
    k0, v0 = kc.t.clone(), vc.t.clone()
    note(f"guard decode {dtype} d={d}")
    bosa.attn_kv_append(kn, vn, kc.t, vc.t, ln, rope_base=10000.0)
    kc.check("k cache")
    vc.check("v cache")
    torch.cuda.synchronize()
    assert ln.cpu().tolist() == [1, 401, Tcap]
    for b, slot in ((0, 0), (1, 400)):
        k0[b, slot] = kc.t[b, slot]
        v0[b, slot] = vc.t[b, slot]
    assert torch.equal(kc.t.cpu(), k0.cpu()) and torch.equal(vc.t.cpu(), v0.cpu()), "append wrote other slots"
    out = Guarded((B, H, d), dtype)
    lse = Guarded((B, H), torch.float32)
    bosa.attn_decode(qn, kc.t, vc.t, ln, out.t, lse.t, rope_base=10000.0, window_left=300)
    out.check("decode out")
    lse.check("decode lse")


def test_elementwise_writes_stay_in_bounds():
    """attn_merge, attn_cast and rope_apply on ragged sizes."""
    B, H, Tq, d = 3, 3, 203, 64
    oa = Guarded((B, Tq, H, d), torch.float32, rnd((B, Tq, H, d), 551, torch.float32))
    la = Guarded((B, H, Tq), torch.float32, rnd((B, H, Tq), 552, torch.float32))
    ob, lb = rnd((B, Tq, H, d), 553, torch.bfloat16), rnd((B, H, Tq), 554, torch.float32)
    note("guard merge / cast / rope_apply")
    bosa.attn_merge(oa.t, la.t, ob, lb)
    oa.check("merge out")
    la.check("merge lse")
    n = 1001
    src = rnd((n,), 555, torch.float32)
    dst = Guarded((n,), torch.bfloat16)
    bosa.attn_cast(src, dst.t)
    dst.check("cast")
    for dt in (torch.bfloat16, torch.float32):
        x = Guarded((B, 77, H, d), dt, rnd((B, 77, H, d), 556, dt))
        bosa.rope_apply(x.t, torch.arange(77, device=DEV) + 5, 10000.0)
        x.check(f"rope_apply {dt}")
