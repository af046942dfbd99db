"""GPU parity of the attention backward (attn_bwd, attn_ring_bwd) against the
fp64 backward oracle, plus its exact properties.

The GPU forward provides out and lse (as a ring step would have them); the
oracle computes the exact gradients of the same bf16 inputs.  Tolerance: the
largest error of a gradient tensor, relative to that tensor's largest
magnitude, must stay below 2e-2.  The kernels round P, dS and the transposed
operands to bf16 (8 significant bits, relative error up to 2^-9 each) before
every matrix product and take delta from the bf16 out; each gradient element
is a sum of such rounded products with mixed signs, so errors of a few 2^-9
relative to the tensor's scale are expected, and 2e-2 (about ten bf16 units)
bounds them with margin, as 2e-2 does for the forward output.
"""
import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
import workloads
from gpu_helpers import DEV, compare, note, np64

pytestmark = pytest.mark.gpu

TOL_G = 2e-2


def rnd(shape, seed, sigma=1.0):
    return workloads.random_normal(shape, seed, torch.bfloat16, sigma)


def run_bwd(q, k, v, dout, *, flags=0, **kw):
    dev = {n: t.to(DEV) for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout))}
    for name in ("kpm", "attn_mask"):
        if kw.get(name) is not None:
            kw[name] = kw[name].to(DEV)
    out, lse = bosa.attn_fwd(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = bosa.attn_bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, flags=flags, **kw)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def ref_bwd(q, k, v, dout, *, q_off=0, kv_off=0, causal=False, kpm=None, attn_mask=None, rope_base=0.0):
    return oracle.attention_backward(np64(q), np64(k), np64(v), np64(dout), q_off=q_off, kv_off=kv_off,
                                     causal=causal, kpm=None if kpm is None else kpm.numpy(),
                                     attn_mask=None if attn_mask is None else attn_mask.numpy(),
                                     rope_base=rope_base, dtype="bf16")


# Floor of the error scale.  Where a row sees a single key, P = 1 and dP
# equals delta, so dS = P (dP - delta) vanishes exactly and so do the terms it
# contributes, while the float32 kernels keep the rounding of a difference of
# two dot products of size |dout| |v| ~ sqrt(d) (unit-variance test inputs),
# about 1e-6 per term.  A gradient element sums n such terms (the keys for
# dq, the queries for dk and dv) with random signs, so its residue grows as
# sqrt(n); a gradient whose reference is below GRAD_FLOOR * sqrt(n) is
# compared against that floor instead of its own size.
GRAD_FLOOR = 1e-4


def compare_grads(got, ref, what):
    errs = []
    n_terms = {"dq": ref[1].shape[1], "dk": ref[0].shape[1], "dv": ref[0].shape[1]}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = np64(g)
        assert g.shape == r.shape, f"{what} {name} shape"
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        floor = GRAD_FLOOR * float(np.sqrt(max(n_terms[name], 1)))
        scale = max(float(np.abs(r).max()) if r.size else 0.0, floor)
        e = float(np.abs(g - r).max()) / scale if r.size else 0.0
        rn = np.sqrt((r ** 2).sum(-1)) + 1e-30
        rel_row = np.sqrt(((g - r) ** 2).sum(-1)) / np.maximum(rn, 1e-3 * scale)
        note(f"  {what} {name}: max|err|/max|ref|={e:.3e} (tol {TOL_G}) max|ref|={scale:.3e} "
             f"row rel L2 max={rel_row.max() if rel_row.size else 0:.2e}")
        errs.append(e)
        assert e <= TOL_G, f"{what} {name}: relative error {e} > {TOL_G}"
    return errs


CASES = [
    # (B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, amask_p, rope, d)
    (1, 1, 1, 1, 0, 0, True, 0.0, 0.0, 0.0, 64),
    (1, 2, 130, 200, 0, 0, False, 0.0, 0.0, 0.0, 128),
    (2, 3, 257, 67, 500, 400, True, 0.0, 0.0, 0.0, 64),
    (1, 2, 300, 300, 0, 0, True, 0.3, 0.0, 10000.0, 128),
    (2, 2, 129, 450, 1000, 700, True, 0.2, 0.1, 10000.0, 128),
    (1, 1, 64, 1000, 70000, 0, False, 0.5, 0.0, 10000.0, 64),
    (1, 2, 200, 333, 0, 100, True, 0.0, 0.0, 500.0, 128),        # rows before the first key: no gradient
    (1, 2, 520, 520, 0, 0, True, 0.0, 0.0, 0.0, 128),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_parity(case):
    B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, am_p, rope, d = CASES[case]
    seed = 7000 + 17 * case
    q = rnd((B, Tq, H, d), seed)
    k = rnd((B, Tkv, H, d), seed + 1)
    v = rnd((B, Tkv, H, d), seed + 2)
    dout = rnd((B, Tq, H, d), seed + 3)
    g = torch.Generator().manual_seed(seed + 4)
    kpm = (torch.rand((B, Tkv), generator=g) < kpm_p).to(torch.uint8) if kpm_p else None
    am = (torch.rand((Tq, Tkv), generator=g) < am_p).to(torch.uint8) if am_p else None
    kw = dict(q_off=q_off, kv_off=kv_off, causal=causal, kpm=kpm, attn_mask=am, rope_base=rope)
    note(f"backward case {case}: B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) causal={causal} "
         f"kpm={kpm_p} amask={am_p} rope={rope} d={d}")
    got = run_bwd(q, k, v, dout, **kw)
    ref = ref_bwd(q, k, v, dout, **kw)
    compare_grads(got, ref, f"case{case}")
    # float32 gradients through ATTN_OUT_F32 agree with the same tolerance
    got32 = run_bwd(q, k, v, dout, flags=bosa.ATTN_OUT_F32, **kw)
    compare_grads(got32, ref, f"case{case} f32")


def test_accumulate_adds_exactly():
    """ATTN_ACCUMULATE adds the float32 gradients into what the buffers hold:
    bitwise the sum of an overwrite run and the previous contents."""
    B, H, T, d = 1, 2, 300, 128
    q, k, v, dout = (rnd((B, T, H, d), 8100 + i) for i in range(4))
    dq0, dk0, dv0 = (rnd((B, T, H, d), 8200 + i).float() for i in range(3))
    for rope in (0.0, 10000.0):
        kw = dict(causal=True, rope_base=rope)
        qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
        out, lse = bosa.attn_fwd(qd, kd, vd, **kw)
        a = bosa.attn_bwd(qd, kd, vd, out, od, lse, flags=bosa.ATTN_OUT_F32, **kw)
        bufs = [dq0.to(DEV), dk0.to(DEV), dv0.to(DEV)]
        bosa.attn_bwd(qd, kd, vd, out, od, lse, *bufs, flags=bosa.ATTN_OUT_F32 | bosa.ATTN_ACCUMULATE, **kw)
        torch.cuda.synchronize()
        for x, base, buf in zip(a, (dq0, dk0, dv0), bufs):
            assert torch.equal(buf.cpu(), base + x.cpu()), f"rope={rope}"


def test_masked_keys_and_empty_rows_exact():
    """Keys excluded by kpm get exactly zero dk, dv; query rows that see no
    key get exactly zero dq; finite garbage in excluded K/V rows changes no
    bit of the gradients."""
    B, H, Tq, Tkv, d = 2, 2, 150, 260, 128
    q = rnd((B, Tq, H, d), 8301)
    k = rnd((B, Tkv, H, d), 8302)
    v = rnd((B, Tkv, H, d), 8303)
    dout = rnd((B, Tq, H, d), 8304)
    g = torch.Generator().manual_seed(8305)
    kpm = (torch.rand((B, Tkv), generator=g) < 0.3).to(torch.uint8)
    kw = dict(causal=True, q_off=0, kv_off=100, kpm=kpm, rope_base=10000.0)
    dq, dk, dv = run_bwd(q, k, v, dout, **kw)
    m = kpm.bool()
    assert torch.all(dk[m] == 0) and torch.all(dv[m] == 0)
    # query rows 0..99 sit before the first key position (100): no allowed key
    assert torch.all(dq[:, :100] == 0)
    k2, v2 = k.clone(), v.clone()
    k2[m] = 1000.0 * k2[m]
    v2[m] = -500.0 * v2[m] + 3.0
    dq2, dk2, dv2 = run_bwd(q, k2, v2, dout, **kw)
    assert torch.equal(dq, dq2)
    assert torch.equal(dk[~m], dk2[~m]) and torch.equal(dv[~m], dv2[~m])


def test_backward_deterministic():
    B, H, T, d = 1, 4, 700, 128
    q, k, v, dout = (rnd((B, T, H, d), 8400 + i) for i in range(4))
    a = run_bwd(q, k, v, dout, causal=True, rope_base=10000.0)
    b = run_bwd(q, k, v, dout, causal=True, rope_base=10000.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_no_tile_skip_is_bit_identical():
    """Skipping future tiles changes no bit of the gradients."""
    B, H, T, d = 1, 2, 400, 64
    q, k, v, dout = (rnd((B, T, H, d), 8500 + i) for i in range(4))
    a = run_bwd(q, k, v, dout, causal=True)
    b = run_bwd(q, k, v, dout, causal=True, flags=bosa.ATTN_NO_TILE_SKIP)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_empty_sides():
    """Tkv = 0: dq = 0; Tq = 0: dk = dv = 0."""
    d = 64
    q = rnd((1, 5, 2, d), 8601).to(DEV)
    k0 = torch.empty((1, 0, 2, d), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.full((1, 2, 5), -float("inf"), device=DEV)
    dq, dk, dv = bosa.attn_bwd(q, k0, k0, out, q, lse)
    torch.cuda.synchronize()
    assert torch.all(dq.cpu() == 0)
    k = rnd((1, 6, 2, d), 8602).to(DEV)
    q0 = torch.empty((1, 0, 2, d), dtype=torch.bfloat16, device=DEV)
    lse0 = torch.empty((1, 2, 0), device=DEV)
    dq, dk, dv = bosa.attn_bwd(q0, k, k, q0, q0, lse0)
    torch.cuda.synchronize()
    assert torch.all(dk.cpu() == 0) and torch.all(dv.cpu() == 0)


def _ring_inputs(w, T, heads, rank):
    P = w.ring_P
    parts = 2 * P if w.zigzag else P
    c = T // parts
    ww = workloads.Workload(**{**w.__dict__, "T": T, "chunk": c})
    k = workloads.draw_tokens(ww, 1, range(parts), heads)
    v = workloads.draw_tokens(ww, 2, range(parts), heads)
    qpos = oracle.local_query_positions(T, P, rank, w.zigzag)
    qchunks = sorted(set((qpos // c).tolist()), key=lambda x: list(qpos // c).index(x))
    q = workloads.draw_tokens(ww, 0, qchunks, heads)
    dout = workloads.draw_tokens(ww, 3, qchunks, heads)
    return q, k, v, dout, qpos


@pytest.mark.parametrize("wi,T,heads,ranks", [(2, 4096, 1, [0, 3]), (4, 8192, 1, [0, 5])])
def test_ring_backward_share(wi, T, heads, ranks):
    """attn_ring_bwd after attn_ring_fwd equals the oracle gradients of the
    share (local rows against every key at absolute positions)."""
    w = workloads.WORKLOADS[wi]
    for rank in ranks:
        q, k, v, dout, qpos = _ring_inputs(w, T, heads, rank)
        note(f"ring backward {w.name} T={T} heads={heads} rank={rank}")
        qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
        out, lse = bosa.attn_ring_fwd(qd, kd, vd, P=w.ring_P, rank=rank, zigzag=w.zigzag, causal=w.causal,
                                      rope_base=w.rope_base)
        dq, dk, dv = bosa.attn_ring_bwd(qd, kd, vd, out, od, lse, P=w.ring_P, rank=rank, zigzag=w.zigzag,
                                        causal=w.causal, rope_base=w.rope_base)
        torch.cuda.synchronize()
        ref = oracle.sdpa_backward(np64(q), np64(k), np64(v), np64(dout), qpos, np.arange(T), causal=w.causal,
                                   rope_base=w.rope_base, dtype="bf16")
        compare_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, f"rank{rank}")


@pytest.mark.parametrize("zigzag,causal", [(True, True), (False, False)])
def test_ring_backward_with_key_padding(zigzag, causal):
    """attn_ring_bwd with a key-padding mask over the whole sequence (one
    batch row padded to a length that ends inside a block, one with random
    holes), RoPE, every rank of P = 4: dq, dk, dv against the oracle."""
    P, B, H, T, d = 4, 2, 2, 1024, 128
    kpm = workloads.random_mask((B, T), 9500 + int(zigzag), 0.15)
    kpm[0, 700:] = 1
    for rank in range(P):
        qpos = oracle.local_query_positions(T, P, rank, zigzag)
        seed = 9510 + 10 * rank + int(zigzag)
        q = rnd((B, T // P, H, d), seed)
        k = rnd((B, T, H, d), seed + 1)
        v = rnd((B, T, H, d), seed + 2)
        dout = rnd((B, T // P, H, d), seed + 3)
        note(f"ring backward kpm: zigzag={zigzag} causal={causal} rank={rank}")
        qd, kd, vd, od, md = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), kpm.to(DEV)
        out, lse = bosa.attn_ring_fwd(qd, kd, vd, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=md,
                                      rope_base=10000.0)
        dq, dk, dv = bosa.attn_ring_bwd(qd, kd, vd, out, od, lse, P=P, rank=rank, zigzag=zigzag, causal=causal,
                                        kpm=md, rope_base=10000.0)
        torch.cuda.synchronize()
        ref = oracle.sdpa_backward(np64(q), np64(k), np64(v), np64(dout), qpos, np.arange(T), causal=causal,
                                   kpm=kpm.numpy(), rope_base=10000.0, dtype="bf16")
        compare_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, f"rank{rank}")


def test_ring_backward_with_a_fully_padded_row():
    """attn_ring_bwd where every key of batch row 1 is padded: that row's
    queries saw no key (out = 0, lse = -inf), so its dq, dk and dv are zero;
    row 0 against the oracle; zigzag, causal, RoPE, every rank of P = 4."""
    P, B, H, T, d = 4, 2, 2, 1024, 128
    kpm = workloads.random_mask((B, T), 9700, 0.2)
    kpm[1, :] = 1
    for rank in range(P):
        qpos = oracle.local_query_positions(T, P, rank, True)
        seed = 9710 + 10 * rank
        q = rnd((B, T // P, H, d), seed)
        k = rnd((B, T, H, d), seed + 1)
        v = rnd((B, T, H, d), seed + 2)
        dout = rnd((B, T // P, H, d), seed + 3)
        note(f"ring backward fully padded row: rank={rank}")
        qd, kd, vd, od, md = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), kpm.to(DEV)
        out, lse = bosa.attn_ring_fwd(qd, kd, vd, P=P, rank=rank, zigzag=True, causal=True, kpm=md, rope_base=10000.0)
        dq, dk, dv = bosa.attn_ring_bwd(qd, kd, vd, out, od, lse, P=P, rank=rank, zigzag=True, causal=True, kpm=md,
                                        rope_base=10000.0)
        torch.cuda.synchronize()
        for g in (dq, dk, dv):
            assert not torch.any(g[1].float().cpu() != 0), "gradient of the padded row"
        ref = oracle.sdpa_backward(np64(q), np64(k), np64(v), np64(dout), qpos, np.arange(T), causal=True,
                                   kpm=kpm.numpy(), rope_base=10000.0, dtype="bf16")
        compare_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, f"rank{rank}")


@pytest.mark.parametrize("causal", [False, True])
def test_batch_rows_with_different_padding(causal):
    """Forward and backward with B*H a multiple of 8 and a key-padding mask
    whose valid length differs per batch row (the workgroups then spread the
    (batch row, head) pairs over the XCDs round-robin): B = 2, H = 4,
    lengths 700 and 230 of 700 keys, against the oracle."""
    B, H, T, d = 2, 4, 700, 128
    kpm = torch.zeros((B, T), dtype=torch.uint8)
    kpm[1, 230:] = 1
    seed = 9800 + int(causal)
    q, k, v, dout = (rnd((B, T, H, d), seed + i) for i in range(4))
    note(f"batch rows with different padding: causal={causal}")
    qd, kd, vd, od, md = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), kpm.to(DEV)
    out, lse = bosa.attn_fwd(qd, kd, vd, causal=causal, kpm=md, rope_base=10000.0)
    dq, dk, dv = bosa.attn_bwd(qd, kd, vd, out, od, lse, causal=causal, kpm=md, rope_base=10000.0,
                               flags=bosa.ATTN_OUT_F32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(np64(q), np64(k), np64(v), causal=causal, kpm=kpm.numpy(), rope_base=10000.0,
                              dtype="bf16")
    compare(out.cpu(), lse.cpu(), ro, rl, "bf16", "forward")
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(dout), causal=causal, kpm=kpm.numpy(),
                                    rope_base=10000.0, dtype="bf16")
    compare_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, "backward")
