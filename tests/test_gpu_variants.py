"""GPU parity of the attention variants against the fp64 oracle: sliding
window and ALiBi bias (attn_fwd_ex), and decoding over a key/value cache
(attn_kv_append, attn_decode).  Tolerances as for the forward: fp32 out and
lse 1e-5; bf16 out 2e-2, lse 1e-3 (max-abs); exclusions bit-exact."""
import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
import workloads
from gpu_helpers import DEV, compare, dt_name, note, np64

pytestmark = pytest.mark.gpu

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def rnd(shape, seed, dtype, sigma=1.0):
    return workloads.random_normal(shape, seed, dtype, sigma)


def run(q, k, v, **kw):
    dev = {n: t.to(DEV) for n, t in (("q", q), ("k", k), ("v", v))}
    for name in ("kpm", "attn_mask", "alibi_slopes"):
        if kw.get(name) is not None:
            kw[name] = kw[name].to(DEV)
    out, lse = bosa.attn_fwd(dev["q"], dev["k"], dev["v"], **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def ref(q, k, v, *, q_off=0, kv_off=0, causal=False, kpm=None, rope_base=0.0, window=None, alibi_slopes=None):
    return oracle.attention(np64(q), np64(k), np64(v), q_off=q_off, kv_off=kv_off, causal=causal,
                            kpm=None if kpm is None else kpm.numpy(), rope_base=rope_base, dtype=dt_name(q),
                            window=(-1, -1) if window is None else window,
                            alibi_slopes=None if alibi_slopes is None else alibi_slopes.double().numpy())


CASES = [
    # (B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, rope, window, alibi, d)
    (1, 2, 300, 300, 0, 0, True, 0.0, 0.0, (100, -1), False, 128),
    (1, 2, 257, 400, 100, 0, False, 0.0, 0.0, (70, 30), False, 64),
    (2, 2, 129, 520, 300, 0, True, 0.2, 10000.0, (128, -1), False, 128),
    (1, 1, 200, 333, 0, 50, False, 0.0, 0.0, (0, 0), False, 128),           # only the aligned diagonal
    (1, 2, 64, 1000, 5000, 4500, False, 0.0, 0.0, (-1, 10), False, 64),     # right edge only
    (1, 3, 300, 300, 0, 0, True, 0.0, 0.0, None, True, 128),
    (2, 2, 190, 450, 200, 0, False, 0.3, 500.0, None, True, 64),
    (1, 2, 130, 700, 600, 0, True, 0.0, 10000.0, (256, -1), True, 128),
    (1, 2, 100, 100, 0, 0, True, 0.0, 0.0, (5000, 5000), False, 128),       # window wider than the sequence
    (1, 1, 64, 256, 0, 1000, True, 0.0, 0.0, (64, -1), False, 64),          # every key after every query
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_variant_parity(case, dtype):
    B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, rope, window, alibi, d = CASES[case]
    dt = DTYPES[dtype]
    seed = 7000 + 13 * case
    q, k, v = rnd((B, Tq, H, d), seed, dt), rnd((B, Tkv, H, d), seed + 1, dt), rnd((B, Tkv, H, d), seed + 2, dt)
    g = torch.Generator().manual_seed(seed + 3)
    kpm = (torch.rand((B, Tkv), generator=g) < kpm_p).to(torch.uint8) if kpm_p > 0 else None
    slopes = workloads.alibi_slopes(H) if alibi else None
    note(f"case {case} {dtype} d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) causal={causal} "
         f"kpm={kpm_p} rope={rope} window={window} alibi={alibi}")
    kw = dict(q_off=q_off, kv_off=kv_off, causal=causal, kpm=kpm, rope_base=rope, window=window, alibi_slopes=slopes)
    out, lse = run(q, k, v, **kw)
    ro, rl = ref(q, k, v, **kw)
    compare(out, lse, ro, rl, dtype, f"case {case}")


def _band_mask(Tq, Tkv, q_off, kv_off, window):
    qp = q_off + np.arange(Tq)[:, None]
    kp = kv_off + np.arange(Tkv)[None, :]
    ok = np.ones((Tq, Tkv), bool)
    if window[0] >= 0:
        ok &= kp >= qp - window[0]
    if window[1] >= 0:
        ok &= kp <= qp + window[1]
    return torch.from_numpy((~ok).astype(np.uint8))


@pytest.mark.parametrize("d", [64, 128])
def test_window_equals_its_attention_mask_bitwise(d):
    """A window skips whole tiles and masks the edge tiles; the same band as
    an attention mask visits every tile masked.  Excluded keys contribute
    exactly zero either way, so the results agree bit for bit; NO_TILE_SKIP
    with the window is bit-identical too, and garbage in keys outside every
    window changes nothing."""
    B, H, Tq, Tkv, q_off, kv_off = 1, 2, 320, 700, 300, 0
    window = (150, 40)
    q, k, v = (rnd((B, T, H, d), 8100 + i, torch.bfloat16) for i, T in enumerate((Tq, Tkv, Tkv)))
    o1, l1 = run(q, k, v, q_off=q_off, kv_off=kv_off, window=window)
    o2, l2 = run(q, k, v, q_off=q_off, kv_off=kv_off, attn_mask=_band_mask(Tq, Tkv, q_off, kv_off, window))
    o3, l3 = run(q, k, v, q_off=q_off, kv_off=kv_off, window=window, flags=bosa.ATTN_NO_TILE_SKIP)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    far = kv_off + np.arange(Tkv) < q_off - window[0]          # before every query's window
    k2, v2 = k.clone(), v.clone()
    k2[:, torch.from_numpy(far)] *= 1000
    v2[:, torch.from_numpy(far)] = 77.0
    o4, l4 = run(q, k2, v2, q_off=q_off, kv_off=kv_off, window=window)
    assert torch.equal(o1, o4) and torch.equal(l1, l4)


def test_alibi_zero_slopes_is_plain_attention_bitwise():
    """Slope 0 adds exactly 0.0 to every score: bit-identical to no ALiBi."""
    B, H, T, d = 1, 2, 300, 128
    q, k, v = (rnd((B, T, H, d), 8200 + i, torch.bfloat16) for i in range(3))
    o1, l1 = run(q, k, v, causal=True)
    o2, l2 = run(q, k, v, causal=True, alibi_slopes=torch.zeros(H))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ decoding
def _ulp_mismatch(a: torch.Tensor, b: torch.Tensor) -> float:
    """Fraction of elements that differ (bf16/fp32 bit patterns)."""
    return float((a != b).float().mean()) if a.numel() else 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rope,window_left,alibi", [(0.0, -1, False), (10000.0, -1, False),
                                                    (10000.0, 300, True)])
def test_decode_steps(dtype, d, rope, window_left, alibi):
    """Prompts of ragged lengths are appended token by token, then each step
    appends one token and decodes it; the caches match the oracle's
    (bit-exact but for rotation ties) and every decoded row matches
    oracle.decode on the same cache."""
    dt = DTYPES[dtype]
    B, H, Tcap = 3, 4, 1200
    prompt = [1, 700, 1100]
    steps = 3
    T = max(prompt) + steps
    seed = 8300 + d + (7 if dtype == "f32" else 0)
    q, k, v = (rnd((B, T, H, d), seed + i, dt) for i in range(3))
    kc = torch.zeros((B, Tcap, H, d), dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    ln = torch.zeros(B, dtype=torch.int32, device=DEV)
    slopes = workloads.alibi_slopes(H) if alibi else None
    # prompt tokens: rows whose prompt is complete are frozen by passing them a full length
    kd, vd = k.to(DEV), v.to(DEV)
    full = torch.full((B,), Tcap, dtype=torch.int32, device=DEV)
    for t in range(max(prompt)):
        active = torch.tensor([t < p for p in prompt], device=DEV)
        lens = torch.where(active, ln, full)
        bosa.attn_kv_append(kd[:, t].contiguous(), vd[:, t].contiguous(), kc, vc, lens, rope_base=rope)
        ln = torch.where(active, lens, ln)
    torch.cuda.synchronize()
    assert ln.cpu().tolist() == prompt
    ref_kc = np.zeros((B, Tcap, H, d))
    ref_vc = np.zeros((B, Tcap, H, d))
    for b in range(B):
        rk, rv, rl = np.zeros((1, Tcap, H, d)), np.zeros((1, Tcap, H, d)), [0]
        for t in range(prompt[b]):
            rk, rv, rl = oracle.kv_append(rk, rv, rl, np64(k[b:b + 1, t]), np64(v[b:b + 1, t]), rope_base=rope,
                                          dtype=dtype)
        assert int(rl[0]) == prompt[b]
        ref_kc[b] = rk[0]
        ref_vc[b] = rv[0]
    note(f"decode {dtype} d={d} rope={rope} window_left={window_left} alibi={alibi} prompts={prompt}")
    mism = _ulp_mismatch(kc.cpu(), torch.from_numpy(ref_kc).to(dt))
    assert mism < 1e-5, f"cached keys differ from the oracle's in {mism:.2e} of the elements"
    assert torch.equal(vc.cpu(), torch.from_numpy(ref_vc).to(dt))
    ref_ln = np.array(prompt)
    for s in range(steps):
        pos = [p + s for p in prompt]
        kn = torch.stack([k[b, pos[b]] for b in range(B)])
        vn = torch.stack([v[b, pos[b]] for b in range(B)])
        qn = torch.stack([q[b, pos[b]] for b in range(B)])
        bosa.attn_kv_append(kn.to(DEV), vn.to(DEV), kc, vc, ln, rope_base=rope)
        out, lse = bosa.attn_decode(qn.to(DEV), kc, vc, ln, rope_base=rope, window_left=window_left,
                                    alibi_slopes=None if slopes is None else slopes.to(DEV))
        torch.cuda.synchronize()
        assert ln.cpu().tolist() == [p + 1 for p in pos]
        # the oracle decodes over its own cache, appended by oracle.kv_append
        ref_kc, ref_vc, ref_ln = oracle.kv_append(ref_kc, ref_vc, ref_ln, np64(kn), np64(vn), rope_base=rope,
                                                  dtype=dtype)
        ro, rl = oracle.decode(np64(qn), ref_kc, ref_vc, ref_ln, rope_base=rope,
                               dtype=dtype, window_left=window_left,
                               alibi_slopes=None if slopes is None else slopes.double().numpy())
        compare(out.cpu()[:, None], lse.cpu()[:, :, None], ro[:, None], rl[:, :, None], dtype, f"step {s}")
    mism = _ulp_mismatch(kc.cpu(), torch.from_numpy(ref_kc).to(dt))
    assert mism < 1e-5, f"cached keys differ from the oracle's in {mism:.2e} of the elements"


def test_decode_full_cache_and_empty_rows():
    """A full row is not written (its length stays Tcap); a row with length 0
    decodes to (0, -inf); lengths beyond Tcap are clamped."""
    B, H, Tcap, d = 3, 2, 100, 128
    dt = torch.bfloat16
    kc = rnd((B, Tcap, H, d), 8400, dt).to(DEV)
    vc = rnd((B, Tcap, H, d), 8401, dt).to(DEV)
    k0, v0 = kc.clone(), vc.clone()
    ln = torch.tensor([Tcap, 0, 40], dtype=torch.int32, device=DEV)
    kn = rnd((B, H, d), 8402, dt).to(DEV)
    vn = rnd((B, H, d), 8403, dt).to(DEV)
    bosa.attn_kv_append(kn, vn, kc, vc, ln)
    torch.cuda.synchronize()
    assert ln.cpu().tolist() == [Tcap, 1, 41]
    assert torch.equal(kc[0], k0[0]) and torch.equal(vc[0], v0[0])
    assert torch.equal(kc[1, 0], kn[1]) and torch.equal(kc[2, 40], kn[2])
    assert torch.equal(kc[1, 1:], k0[1, 1:]) and torch.equal(kc[2, 41:], k0[2, 41:])
    lens = torch.tensor([0, Tcap + 50, 1], dtype=torch.int32, device=DEV)
    q = rnd((B, H, d), 8404, dt)
    out, lse = bosa.attn_decode(q.to(DEV), kc, vc, lens)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.all(out[0] == 0) and torch.all(lse[0] == -np.inf)
    ro, rl = oracle.decode(np64(q), np64(kc.cpu()), np64(vc.cpu()), [0, Tcap, 1], dtype="bf16")
    compare(out[:, None], lse[:, :, None], ro[:, None], rl[:, :, None], "bf16", "clamped lengths")
    # a single visible slot: out is that slot's value exactly
    assert torch.equal(out[2], vc[2, 0].cpu())


def test_decode_long_cache_sampled():
    """A long ragged cache (the decode workload's shape at reduced batch):
    every row against the oracle."""
    B, H, Tcap, d = 2, 4, 32768, 128
    dt = torch.bfloat16
    kc = rnd((B, Tcap, H, d), 8500, dt).to(DEV)
    vc = rnd((B, Tcap, H, d), 8501, dt).to(DEV)
    lens = torch.tensor([32768, 17001], dtype=torch.int32, device=DEV)
    q = rnd((B, H, d), 8502, dt)
    slopes = workloads.alibi_slopes(H)
    for kw in (dict(), dict(rope_base=10000.0), dict(window_left=4095, alibi_slopes=slopes)):
        dkw = dict(kw)
        if "alibi_slopes" in dkw:
            dkw["alibi_slopes"] = dkw["alibi_slopes"].to(DEV)
        out, lse = bosa.attn_decode(q.to(DEV), kc, vc, lens, **dkw)
        torch.cuda.synchronize()
        rkw = dict(kw)
        if "alibi_slopes" in rkw:
            rkw["alibi_slopes"] = rkw["alibi_slopes"].double().numpy()
        ro, rl = oracle.decode(np64(q), np64(kc.cpu()), np64(vc.cpu()), lens.cpu().numpy(), dtype="bf16", **rkw)
        compare(out.cpu()[:, None], lse.cpu()[:, :, None], ro[:, None], rl[:, :, None], "bf16", f"long {kw.keys()}")


# ------------------------------------------------------------------ backward with variants
BWD_CASES = [
    # (B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, rope, window, alibi, d)
    (1, 2, 300, 300, 0, 0, True, 0.0, 0.0, (100, -1), False, 128),
    (1, 2, 257, 400, 100, 0, False, 0.0, 0.0, (70, 30), False, 64),
    (1, 2, 200, 333, 0, 50, False, 0.0, 0.0, (0, 0), False, 128),
    (1, 3, 300, 300, 0, 0, True, 0.0, 0.0, None, True, 128),
    (2, 2, 190, 450, 200, 0, False, 0.3, 500.0, None, True, 64),
    (1, 2, 130, 700, 600, 0, True, 0.0, 10000.0, (256, -1), True, 128),
    (1, 2, 64, 1000, 5000, 4500, False, 0.0, 0.0, (-1, 10), True, 128),
    (1, 1, 64, 256, 0, 1000, True, 0.0, 0.0, (64, -1), False, 64),     # every key after every query
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_variant_backward_parity(case):
    """attn_bwd_ex against the fp64 backward oracle with the same window and
    slopes: the largest error of each gradient relative to that gradient's
    largest magnitude within 2e-2 (as for the plain backward)."""
    B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, rope, window, alibi, d = BWD_CASES[case]
    seed = 9000 + 17 * case
    dt = torch.bfloat16
    q, k, v = rnd((B, Tq, H, d), seed, dt), rnd((B, Tkv, H, d), seed + 1, dt), rnd((B, Tkv, H, d), seed + 2, dt)
    dout = rnd((B, Tq, H, d), seed + 3, dt)
    g = torch.Generator().manual_seed(seed + 4)
    kpm = (torch.rand((B, Tkv), generator=g) < kpm_p).to(torch.uint8) if kpm_p > 0 else None
    slopes = workloads.alibi_slopes(H) if alibi else None
    note(f"bwd case {case} d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) causal={causal} "
         f"kpm={kpm_p} rope={rope} window={window} alibi={alibi}")
    kw = dict(q_off=q_off, kv_off=kv_off, causal=causal, rope_base=rope, window=window)
    dev = {n: t.to(DEV) for n, t in (("q", q), ("k", k), ("v", v), ("dout", dout))}
    dkw = dict(kw, kpm=None if kpm is None else kpm.to(DEV), alibi_slopes=None if slopes is None else slopes.to(DEV))
    out, lse = bosa.attn_fwd(dev["q"], dev["k"], dev["v"], **dkw)
    grads = bosa.attn_bwd(dev["q"], dev["k"], dev["v"], out, dev["dout"], lse, **dkw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(np64(q), np64(k), np64(v), np64(dout), q_off=q_off, kv_off=kv_off,
                                    causal=causal, kpm=None if kpm is None else kpm.numpy(), rope_base=rope,
                                    dtype="bf16", window=(-1, -1) if window is None else window,
                                    alibi_slopes=None if slopes is None else slopes.double().numpy())
    for name, gg, r in zip(("dq", "dk", "dv"), grads, ref):
        gv = np64(gg.cpu())
        assert np.all(np.isfinite(gv)), f"{name}: non-finite"
        scale = float(np.abs(r).max()) if r.size else 0.0
        if scale == 0.0:
            # every row sees at most one key, so dS = P (dP - delta) cancels to
            # exactly zero in the oracle; the kernels round dP and delta
            # differently, which leaves float32 noise of the order of 1e-7
            big = float(np.abs(gv).max())
            note(f"  {name}: reference exactly zero, max|got| = {big:.2e}")
            assert big <= 1e-5, f"{name}: {big}"
            continue
        e = float(np.abs(gv - r).max()) / scale
        note(f"  {name}: max|err|/max|ref| = {e:.3e}")
        assert e <= 2e-2, f"{name}: relative error {e}"


def test_huge_windows_are_no_limit():
    """Windows wider than any position difference (up to 2^63 - 1) exclude
    nothing: the results equal the call without a window bit for bit, in
    the forward, the backward and decoding."""
    B, H, T, d = 1, 2, 200, 128
    big = (1 << 63) - 1
    q, k, v = (rnd((B, T, H, d), 9500 + i, torch.bfloat16) for i in range(3))
    o1, l1 = run(q, k, v, causal=True, q_off=1000, kv_off=900)
    o2, l2 = run(q, k, v, causal=True, q_off=1000, kv_off=900, window=(big, big))
    o3, l3 = run(q, k, v, causal=False, window=(big, -1))
    o4, l4 = run(q, k, v, causal=False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    kc = rnd((1, 300, H, d), 9510, torch.bfloat16).to(DEV)
    vc = rnd((1, 300, H, d), 9511, torch.bfloat16).to(DEV)
    ln = torch.tensor([257], dtype=torch.int32, device=DEV)
    qn = rnd((1, H, d), 9512, torch.bfloat16).to(DEV)
    a, la = bosa.attn_decode(qn, kc, vc, ln, window_left=big)
    b2, lb = bosa.attn_decode(qn, kc, vc, ln)
    torch.cuda.synchronize()
    assert torch.equal(a, b2) and torch.equal(la, lb)


# ------------------------------------------------------------------ ring shares with variants
def _ring_share_inputs(w, T, heads, rank):
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


@pytest.mark.parametrize("wi,T,rank,window,alibi", [
    (2, 4096, 3, (700, -1), False),
    (2, 4096, 2, (300, -1), True),
    (4, 8192, 0, (1000, -1), True),
    (4, 8192, 5, (3000, -1), False),
])
def test_ring_share_with_window(wi, T, rank, window, alibi):
    """attn_ring_fwd_ex / attn_ring_bwd_ex: the share's rows against every key
    at absolute positions with the window and penalty equal the oracle's; the
    executor issues fewer attention launches than the full plan (sub-calls
    whose key block lies outside every row's window are not issued)."""
    w = workloads.WORKLOADS[wi]
    heads = 2
    q, k, v, dout, qpos = _ring_share_inputs(w, T, heads, rank)
    slopes = workloads.alibi_slopes(heads) if alibi else None
    note(f"ring {w.name} T={T} rank={rank} window={window} alibi={alibi}")
    qd, kd, vd, od = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    sd = None if slopes is None else slopes.to(DEV)
    n_plan = len(bosa.attn_ring_plan(T, w.ring_P, rank, w.zigzag, w.causal))
    with bosa.KernelTimer(256) as kt:
        out, lse = bosa.attn_ring_fwd(qd, kd, vd, P=w.ring_P, rank=rank, zigzag=w.zigzag, causal=w.causal,
                                      rope_base=w.rope_base, window=window, alibi_slopes=sd)
        torch.cuda.synchronize()
    note(f"  {len(kt.ms)} attention launches of {n_plan} sub-calls in the plan")
    assert 0 < len(kt.ms) < n_plan
    ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=w.causal, rope_base=w.rope_base,
                         dtype="bf16", window=window, alibi_slopes=None if slopes is None else slopes.double().numpy())
    compare(out.cpu(), lse.cpu(), ro, rl, "bf16", "forward")
    grads = bosa.attn_ring_bwd(qd, kd, vd, out, od, lse, P=w.ring_P, rank=rank, zigzag=w.zigzag, causal=w.causal,
                               rope_base=w.rope_base, window=window, alibi_slopes=sd)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(np64(q), np64(k), np64(v), np64(dout), qpos, np.arange(T), causal=w.causal,
                               rope_base=w.rope_base, dtype="bf16", window=window,
                               alibi_slopes=None if slopes is None else slopes.double().numpy())
    for name, gg, r in zip(("dq", "dk", "dv"), grads, ref):
        gv = np64(gg.cpu())
        e = float(np.abs(gv - r).max()) / float(np.abs(r).max())
        note(f"  {name}: max|err|/max|ref| = {e:.3e}")
        assert np.all(np.isfinite(gv)) and e <= 2e-2, f"{name}: relative error {e}"
