"""GPU parity of the HIP path against the fp64 oracle (C ABI via ctypes).

Sizes here are ones the oracle finishes in seconds while spanning several
128-row query tiles and 64-key tiles with ragged tails.  Inputs are seeded
draws rounded to the input dtype; the oracle sees exactly those values.
"""
import json
import os

import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
import workloads
from gpu_helpers import DEV, chained_ring_reference, compare, dt_name, gpu_fwd, note, np64, ref_fwd

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, dtype, sigma=1.0):
    return workloads.random_normal(shape, seed, dtype, sigma)


# ------------------------------------------------------------------ printed example
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_worked_example_exact(dtype, d):
    """Transformers and Attention #24: scores [0,0], values [2,0],[0,4] ->
    [1,2]; excluding source 2 -> [2,0].  Exact in both dtypes."""
    g = json.load(open(os.path.join(GOLDEN, "sdpa_worked_example.json")))
    q = torch.zeros((1, 1, 1, d), dtype=dtype)
    k = rnd((1, 2, 1, d), 1, dtype)
    v = torch.zeros((1, 2, 1, d), dtype=dtype)
    v[0, :, 0, :2] = torch.tensor(g["values"], dtype=dtype)
    out, lse = gpu_fwd(q, k, v)
    assert out[0, 0, 0, :2].float().tolist() == g["both_sources"]["out"]
    assert torch.all(out[0, 0, 0, 2:] == 0)
    assert abs(float(lse[0, 0, 0]) - g["both_sources"]["lse"]) <= 1e-6
    out, lse = gpu_fwd(q, k, v, kpm=torch.tensor([[0, 1]], dtype=torch.uint8))
    assert out[0, 0, 0, :2].float().tolist() == g["second_source_excluded"]["out"]
    assert float(lse[0, 0, 0]) == g["second_source_excluded"]["lse"]


# ------------------------------------------------------------------ general parity
CASES = [
    # (B, H, Tq, Tkv, q_off, kv_off, causal, kpm_p, amask_p, rope)
    (1, 1, 1, 1, 0, 0, True, 0.0, 0.0, 0.0),
    (1, 2, 130, 200, 0, 0, False, 0.0, 0.0, 0.0),
    (2, 3, 257, 67, 500, 400, True, 0.0, 0.0, 0.0),
    (1, 2, 300, 300, 0, 0, True, 0.3, 0.0, 10000.0),
    (2, 2, 129, 450, 1000, 700, True, 0.2, 0.1, 10000.0),
    (1, 1, 64, 1000, 70000, 0, False, 0.5, 0.0, 10000.0),
    (1, 2, 200, 333, 0, 100, True, 0.0, 0.0, 500.0),        # rows before the first key: empty
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_parity_small(dtype, d, case):
    B, H, Tq, Tkv, q_off, kv_off, causal, kp, ap, rope = CASES[case]
    seed = 100 * case + d
    note(f"case {case} dtype={dtype} d={d} B={B} H={H} Tq={Tq} Tkv={Tkv} offs=({q_off},{kv_off}) causal={causal}")
    q, k, v = rnd((B, Tq, H, d), seed, dtype), rnd((B, Tkv, H, d), seed + 1, dtype), rnd((B, Tkv, H, d), seed + 2, dtype)
    kpm = workloads.random_mask((B, Tkv), seed + 3, kp) if kp else None
    am = workloads.random_mask((Tq, Tkv), seed + 4, ap) if ap else None
    kw = dict(q_off=q_off, kv_off=kv_off, causal=causal, kpm=kpm, attn_mask=am, rope_base=rope)
    out, lse = gpu_fwd(q, k, v, **kw)
    ro, rl = ref_fwd(q, k, v, **kw)
    compare(out, lse, ro, rl, "f32" if dtype == torch.float32 else "bf16", f"case{case}")


# ------------------------------------------------------------------ workloads 0 and 1 in full
def test_workload0_fp32_full():
    w = workloads.WORKLOADS[0]
    q, k, v = (workloads.draw_tokens(w, t, [0]) for t in (0, 1, 2))
    out, lse = gpu_fwd(q, k, v, causal=True)
    ro, rl = ref_fwd(q, k, v, causal=True)
    compare(out, lse, ro, rl, "f32", w.name)


def test_workload1_gpt2s_full():
    w = workloads.WORKLOADS[1]
    q, k, v = (workloads.draw_tokens(w, t, [0]) for t in (0, 1, 2))
    kpm = workloads.key_padding_mask(w)
    out, lse = gpu_fwd(q, k, v, causal=True, kpm=kpm)
    ro, rl = ref_fwd(q, k, v, causal=True, kpm=kpm)
    compare(out, lse, ro, rl, "bf16", w.name)


# ------------------------------------------------------------------ ring shares, reduced heads
def _ring_case(w, heads, T=None, rank=None):
    T = w.T if T is None else T
    P = w.ring_P
    rank = w.ring_rank if rank is None else rank
    parts = 2 * P if w.zigzag else P
    c = T // parts
    # draw per-chunk with the workload's seeds, at chunk size c
    ww = workloads.Workload(**{**w.__dict__, "T": T, "chunk": c, "H": w.H})
    k = workloads.draw_tokens(ww, 1, range(parts), heads)
    v = workloads.draw_tokens(ww, 2, range(parts), heads)
    qpos = oracle.local_query_positions(T, P, rank, w.zigzag)
    qchunks = sorted(set((qpos // c).tolist()), key=lambda x: list(qpos // c).index(x))
    q = workloads.draw_tokens(ww, 0, qchunks, heads)
    return q, k, v, qpos


@pytest.mark.parametrize("wi,T,heads,ranks", [(2, 8192, 2, [3]), (2, 4096, 1, [0, 1, 2, 3]),
                                              (4, 8192, 2, list(range(8))), (4, 16384, 1, [0, 7])])
def test_ring_share_reduced(wi, T, heads, ranks):
    w = workloads.WORKLOADS[wi]
    for rank in ranks:
        q, k, v, qpos = _ring_case(w, heads, T, rank)
        note(f"ring {w.name} T={T} heads={heads} rank={rank}")
        out, lse = bosa.attn_ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P=w.ring_P, rank=rank, zigzag=w.zigzag,
                                      causal=w.causal, rope_base=w.rope_base)
        torch.cuda.synchronize()
        ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=w.causal,
                             rope_base=w.rope_base, dtype="bf16")
        compare(out.cpu(), lse.cpu(), ro, rl, "bf16", f"rank{rank}")


# ------------------------------------------------------------------ masking is bit-exact
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_masked_keys_bit_exact(dtype):
    """Finite garbage in K/V at masked positions changes no bit (padding,
    attention mask and causal exclusions); kpm written as an attention mask
    gives identical bits; visiting every tile (NO_TILE_SKIP) gives identical
    bits."""
    B, H, Tq, Tkv, d = 2, 2, 200, 333, 128
    q, k, v = rnd((B, Tq, H, d), 1, dtype), rnd((B, Tkv, H, d), 2, dtype), rnd((B, Tkv, H, d), 3, dtype)
    kpm = workloads.random_mask((B, Tkv), 4, 0.3)
    kpm[:, 250:] = 1
    kw = dict(q_off=100, kv_off=0, causal=True, kpm=kpm, rope_base=10000.0)
    o1, l1 = gpu_fwd(q, k, v, **kw)
    k2, v2 = k.clone(), v.clone()
    bad = kpm.bool()
    k2[bad] = (k2[bad].float() * 1000).to(dtype)
    v2[bad] = torch.full_like(v2[bad], 1000)
    # keys after every query's causal limit (position > 100 + 199) are masked too
    k2[:, 300:] = 77
    v2[:, 300:] = -500
    o2, l2 = gpu_fwd(q, k2, v2, **kw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = gpu_fwd(q, k, v, **kw, flags=bosa.ATTN_NO_TILE_SKIP)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # per batch item the padding mask equals an attention mask with those columns set
    for b in range(B):
        kwb = dict(kw)
        kwb.pop("kpm")
        am = kpm[b].unsqueeze(0).expand(Tq, Tkv).contiguous()
        ob, lb = gpu_fwd(q[b:b + 1], k[b:b + 1], v[b:b + 1], attn_mask=am, **kwb)
        assert torch.equal(ob[0], o1[b]) and torch.equal(lb[0], l1[b])


def test_value_probes_identity_and_ones():
    """V = I makes out the probability rows: masked and future entries are
    exactly 0; V = 1 gives rows summing to 1."""
    B, H, T, d = 1, 2, 100, 128
    q, k = rnd((B, T, H, d), 5, torch.bfloat16), rnd((B, T, H, d), 6, torch.bfloat16)
    kpm = workloads.random_mask((B, T), 7, 0.2)
    kpm[0, 0] = 0
    v = torch.zeros((B, T, H, d), dtype=torch.bfloat16)
    for j in range(T):
        v[0, j, :, j] = 1
    out, lse = gpu_fwd(q, k, v, causal=True, kpm=kpm)
    P = out[0, :, :, :T].float()                        # (Tq, H, Tkv)
    allowed = torch.ones(T, T, dtype=torch.bool).tril() & (kpm[0] == 0)[None, :]
    assert torch.all(P.permute(1, 0, 2)[:, ~allowed] == 0)
    ro, rl = ref_fwd(q, k, v, causal=True, kpm=kpm)
    compare(out, lse, ro, rl, "bf16", "V=I")
    ones = torch.ones_like(v)
    out, _ = gpu_fwd(q, k, ones, causal=True, kpm=kpm)
    assert float((out.float() - 1).abs().max()) <= 2e-2


# ------------------------------------------------------------------ fused vs standalone
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_merge_matches_standalone_merge_bitwise(dtype):
    B, H, Tq, d = 1, 3, 190, 128
    q = rnd((B, Tq, H, d), 10, dtype).to(DEV)
    ka, va = rnd((B, 150, H, d), 11, dtype).to(DEV), rnd((B, 150, H, d), 12, dtype).to(DEV)
    kb, vb = rnd((B, 99, H, d), 13, dtype).to(DEV), rnd((B, 99, H, d), 14, dtype).to(DEV)
    kw = dict(q_off=200, causal=True, rope_base=10000.0, flags=bosa.ATTN_OUT_F32)
    oa, la = bosa.attn_fwd(q, ka, va, kv_off=150, **kw)
    ob, lb = bosa.attn_fwd(q, kb, vb, kv_off=0, **kw)
    fo, fl = oa.clone(), la.clone()
    bosa.attn_fwd(q, kb, vb, fo, fl, kv_off=0, q_off=200, causal=True, rope_base=10000.0,
                  flags=bosa.ATTN_OUT_F32 | bosa.ATTN_ACCUMULATE)
    so, sl = oa.clone(), la.clone()
    bosa.attn_merge(so, sl, ob, lb)
    torch.cuda.synchronize()
    assert torch.equal(fo, so) and torch.equal(fl, sl)
    # commutativity and the (0, -inf) identity, bit for bit
    to, tl = ob.clone(), lb.clone()
    bosa.attn_merge(to, tl, oa, la)
    zo, zl = torch.zeros_like(oa), torch.full_like(la, float("-inf"))
    io, il = oa.clone(), la.clone()
    bosa.attn_merge(io, il, zo, zl)
    torch.cuda.synchronize()
    assert torch.equal(to, so) and torch.equal(tl, sl)
    assert torch.equal(io, oa) and torch.equal(il, la)
    # against the oracle merge of the oracle partials
    qc = q.cpu()
    ra = ref_fwd(qc, ka.cpu(), va.cpu(), q_off=200, kv_off=150, causal=True, rope_base=10000.0)
    rb = ref_fwd(qc, kb.cpu(), vb.cpu(), q_off=200, kv_off=0, causal=True, rope_base=10000.0)
    ro, rl = oracle.merge(*ra, *rb)
    compare(so.cpu(), sl.cpu(), ro, rl, "f32" if dtype == torch.float32 else "bf16", "merge")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_rope_matches_rope_apply_bitwise(dtype):
    """RoPE fused into the Q/K load gives the same bits as rotating the
    stored tensors with rope_apply and attending without RoPE."""
    B, H, Tq, Tkv, d = 2, 2, 150, 260, 64
    q, k, v = rnd((B, Tq, H, d), 20, dtype), rnd((B, Tkv, H, d), 21, dtype), rnd((B, Tkv, H, d), 22, dtype)
    q_off, kv_off = 100000, 99900
    o1, l1 = gpu_fwd(q, k, v, q_off=q_off, kv_off=kv_off, causal=True, rope_base=10000.0)
    qd, kd = q.to(DEV), k.to(DEV)
    bosa.rope_apply(qd, torch.arange(q_off, q_off + Tq, device=DEV), 10000.0)
    bosa.rope_apply(kd, torch.arange(kv_off, kv_off + Tkv, device=DEV), 10000.0)
    o2, l2 = gpu_fwd(qd.cpu(), kd.cpu(), v, q_off=q_off, kv_off=kv_off, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # rope_apply against the oracle's rotation (float64, rounded once to the
    # dtype): the same bits except where the two float64 angle evaluations
    # (about 1e-11 rad apart at positions near 1e5) land on opposite sides of
    # a rounding midpoint, then one unit apart: a rate of about 1e-11 / 2^-24
    # for float32, about 1e-11 / 2^-8 (none expected) for bf16
    ref = oracle.round_to_dtype(oracle.rope_rotate(np64(q), q_off + np.arange(Tq), 10000.0),
                                "f32" if dtype == torch.float32 else "bf16")
    got = np64(qd.cpu())
    diff = got != ref
    note(f"rope_apply {dtype}: {int(diff.sum())} of {diff.size} elements differ from the oracle")
    assert diff.mean() < (2e-4 if dtype == torch.float32 else 1e-5)
    ulp = 2.0 ** -23 if dtype == torch.float32 else 2.0 ** -7
    assert np.all(np.abs(got - ref)[diff] <= np.abs(ref[diff]) * ulp)


def test_deterministic():
    B, H, T, d = 1, 4, 700, 128
    q, k, v = (rnd((B, T, H, d), 30 + i, torch.bfloat16) for i in range(3))
    kpm = workloads.random_mask((B, T), 33, 0.1)
    a = gpu_fwd(q, k, v, causal=True, kpm=kpm, rope_base=10000.0)
    b = gpu_fwd(q, k, v, causal=True, kpm=kpm, rope_base=10000.0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_and_degenerate_inputs():
    dtype = torch.bfloat16
    q = rnd((1, 5, 2, 64), 40, dtype)
    k = rnd((1, 0, 2, 64), 41, dtype)
    out, lse = gpu_fwd(q, k, k)
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))
    # everything padded
    k = rnd((1, 70, 2, 64), 42, dtype)
    out, lse = gpu_fwd(q, k, k, kpm=torch.ones((1, 70), dtype=torch.uint8))
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))
    # Tq = 0 is a no-op
    o, l = gpu_fwd(q[:, :0], k, k)
    assert o.shape == (1, 0, 2, 64)


@pytest.mark.parametrize("order", ["ring", "reversed", "random"])
@pytest.mark.parametrize("chunk", [64, 256, 1000])
def test_block_order_and_size_invariance(order, chunk):
    """Splitting K/V into blocks of any size, visited in any order and merged
    with ACCUMULATE, matches the oracle's one-block result."""
    B, H, Tq, T, d = 1, 2, 256, 2000, 128
    q = rnd((B, Tq, H, d), 50, torch.bfloat16)
    k, v = rnd((B, T, H, d), 51, torch.bfloat16), rnd((B, T, H, d), 52, torch.bfloat16)
    q_off = T - Tq
    starts = list(range(0, T, chunk))
    if order == "reversed":
        starts = starts[::-1]
    elif order == "random":
        starts = list(np.random.default_rng(3).permutation(starts))
    else:  # own block first, then earlier ones
        own = max(s for s in starts if s <= q_off)
        starts = [own] + [s for s in sorted(starts, reverse=True) if s != own]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    acc = torch.empty((B, Tq, H, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=DEV)
    for i, s in enumerate(starts):
        e = min(s + chunk, T)
        fl = bosa.ATTN_OUT_F32 | (bosa.ATTN_ACCUMULATE if i else 0)
        bosa.attn_fwd(qd, kd[:, s:e].contiguous(), vd[:, s:e].contiguous(), acc, lse, q_off=q_off, kv_off=int(s),
                      causal=True, rope_base=10000.0, flags=fl)
    torch.cuda.synchronize()
    ro, rl = ref_fwd(q, k, v, q_off=q_off, causal=True, rope_base=10000.0)
    compare(acc.cpu(), lse.cpu(), ro, rl, "bf16", f"{order}/{chunk}")


# ------------------------------------------------------------------ ring shares with key padding
RING_KPM_CASES = [
    # (P, zigzag, causal, dtype, d)
    (4, False, False, torch.bfloat16, 128),
    (4, True, True, torch.bfloat16, 64),
    (2, True, True, torch.float32, 128),
    (4, False, True, torch.float32, 64),
]


@pytest.mark.parametrize("case", range(len(RING_KPM_CASES)))
def test_ring_share_with_key_padding(case):
    """attn_ring_fwd with a key-padding mask over the whole sequence (each
    sub-call sees the mask at its block's keys): two batch rows, one padded
    to a valid length that ends inside a block, one with random holes, RoPE,
    every rank, against the oracle over every key."""
    P, zigzag, causal, dtype, d = RING_KPM_CASES[case]
    B, H, T = 2, 2, 1536
    kpm = workloads.random_mask((B, T), 9400 + case, 0.15)
    kpm[0, 1000:] = 1
    for rank in range(P):
        qpos = oracle.local_query_positions(T, P, rank, zigzag)
        seed = 9410 + 10 * case + rank
        q = rnd((B, T // P, H, d), seed, dtype)
        k = rnd((B, T, H, d), seed + 100, dtype)
        v = rnd((B, T, H, d), seed + 200, dtype)
        note(f"ring kpm case {case}: P={P} zigzag={zigzag} causal={causal} {dtype} d={d} rank={rank}")
        out, lse = bosa.attn_ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P=P, rank=rank, zigzag=zigzag, causal=causal,
                                      kpm=kpm.to(DEV), rope_base=10000.0)
        torch.cuda.synchronize()
        ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=causal, kpm=kpm.numpy(),
                             rope_base=10000.0, dtype=dt_name(q))
        compare(out.cpu(), lse.cpu(), ro, rl, dt_name(q), f"rank{rank}")


@pytest.mark.parametrize("Tq,Tkv,q_off,kp,rope", [(1000, 1000, 0, 0.0, 0.0), (650, 900, 250, 0.2, 10000.0),
                                                 (300, 300, 0, 0.0, 0.0)])
def test_paired_query_units_equal_unpaired_bitwise(Tq, Tkv, q_off, kp, rope):
    """A causal bf16 attn_fwd whose workgroups all run at once (at most one
    per CU) pairs 128-row query units: workgroup t takes units t and n - 1 - t
    (300 rows: three units, the middle one alone).  With more workgroups than
    CUs each keeps 256 consecutive rows.  A row's result does not depend on
    which workgroup computes it: one head alone against the same head
    repeated until the grid exceeds the CU count, bit for bit."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    d, bf = 128, torch.bfloat16
    q = rnd((1, Tq, 1, d), 9701, bf)
    k = rnd((1, Tkv, 1, d), 9702, bf)
    v = rnd((1, Tkv, 1, d), 9703, bf)
    kpm = workloads.random_mask((1, Tkv), 9704, kp).to(DEV) if kp else None
    H = n_cu // ((Tq + 255) // 256) + 1
    note(f"paired vs unpaired: Tq={Tq} Tkv={Tkv} q_off={q_off} kpm={kp} rope={rope}: 1 head, then {H} heads")
    o1, l1 = bosa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), q_off=q_off, causal=True, kpm=kpm, rope_base=rope)
    rep = lambda x: x.expand(1, x.shape[1], H, d).contiguous().to(DEV)
    oH, lH = bosa.attn_fwd(rep(q), rep(k), rep(v), q_off=q_off, causal=True, kpm=kpm, rope_base=rope)
    torch.cuda.synchronize()
    for h in (0, H // 2, H - 1):
        assert torch.equal(oH[:, :, h:h + 1].view(torch.int16).cpu(), o1.view(torch.int16).cpu()), f"head {h}: out"
        assert torch.equal(lH[:, h:h + 1].cpu(), l1.cpu()), f"head {h}: lse"


@pytest.mark.parametrize("zigzag,causal,kp,rope,d", [(True, True, 0.0, 10000.0, 128), (False, True, 0.2, 10000.0, 128),
                                                    (True, False, 0.2, 0.0, 64), (False, False, 0.0, 500.0, 64)])
def test_ring_share_equals_its_subcalls_bitwise(zigzag, causal, kp, rope, d):
    """attn_ring_fwd runs each query block's sub-calls chained in one launch,
    the softmax state carried across them; its out and lse equal, bit for bit,
    one attn_fwd call per launch over that launch's keys in ring order (causal
    order as an attention mask, rotations applied beforehand), merged into a
    float32 accumulator per query block and cast, and match one attn_fwd call
    per sub-call of attn_ring_plan up to rounding, on every rank."""
    _ring_share_vs_subcalls(4, 1, 2, 1536, d, zigzag, causal, kp, rope, range(4))


@pytest.mark.parametrize("zigzag,T", [(False, 18432), (True, 36864)])
def test_ring_share_equals_its_subcalls_bitwise_above_one_round(zigzag, T):
    """The same checks where a launch has more workgroups than the chip has
    CUs (16 heads x 18 query tiles = 288): there a chain ends after the
    sub-call that causal order cuts through the query block, so a query block
    takes several launches that merge into its float32 partial, the last one
    writing the final output; ranks 0 and 3 of P = 4, key padding, RoPE."""
    _ring_share_vs_subcalls(4, 1, 16, T, 128, zigzag, True, 0.1, 10000.0, (0, 3))


def _ring_share_vs_subcalls(P, B, H, T, d, zigzag, causal, kp, rope, ranks):
    k = rnd((B, T, H, d), 9601, torch.bfloat16).to(DEV)
    v = rnd((B, T, H, d), 9602, torch.bfloat16).to(DEV)
    kpm = workloads.random_mask((B, T), 9603, kp).to(DEV) if kp else None
    for rank in ranks:
        q = rnd((B, T // P, H, d), 9610 + rank, torch.bfloat16).to(DEV)
        out, lse = bosa.attn_ring_fwd(q, k, v, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=kpm, rope_base=rope)
        plan = bosa.attn_ring_plan(T, P, rank, zigzag, causal)
        note(f"ring = chained sub-calls: zigzag={zigzag} causal={causal} kpm={kp} rope={rope} d={d} rank={rank}: "
             f"{len(plan)} sub-calls")
        ro, rl = chained_ring_reference(q, k, v, kpm, P, rank, zigzag, causal, rope)
        assert torch.equal(out.view(torch.int16).cpu(), ro.view(torch.int16).cpu()), f"rank {rank}: out"
        assert torch.equal(lse.cpu(), rl.cpu()), f"rank {rank}: lse"
        # and against one attn_fwd call per sub-call (partials merged after
        # every sub-call): the same result up to rounding
        parts = {}
        for e in plan:
            r0, nr, k0, nk = e.q_row0, e.q_rows, e.kv_pos0, e.kv_rows
            if r0 not in parts:
                parts[r0] = (torch.empty((B, nr, H, d), dtype=torch.float32, device=DEV),
                             torch.empty((B, H, nr), dtype=torch.float32, device=DEV))
            acc, ls = parts[r0]
            flags = bosa.ATTN_OUT_F32 | (bosa.ATTN_ACCUMULATE if e.accumulate else 0)
            bosa.attn_fwd(q[:, r0:r0 + nr].contiguous(), k[:, k0:k0 + nk].contiguous(), v[:, k0:k0 + nk].contiguous(),
                          acc, ls, q_off=e.q_pos0, kv_off=k0, causal=causal,
                          kpm=None if kpm is None else kpm[:, k0:k0 + nk].contiguous(), rope_base=rope, flags=flags)
        torch.cuda.synchronize()
        for r0, (acc, ls) in parts.items():
            nr = acc.shape[1]
            eo = float((out[:, r0:r0 + nr].float() - acc).abs().max())
            fin = torch.isfinite(ls)
            assert torch.equal(fin, torch.isfinite(lse[:, :, r0:r0 + nr])), f"rank {rank} rows {r0}: empty rows"
            el = float((lse[:, :, r0:r0 + nr][fin] - ls[fin]).abs().max()) if bool(fin.any()) else 0.0
            assert eo <= 8e-3 and el <= 2e-5, f"rank {rank} rows {r0}: out {eo} lse {el} against the sub-calls"
        # every tile visited and masked instead of skipped: the same bits
        o2, l2 = bosa.attn_ring_fwd(q, k, v, P=P, rank=rank, zigzag=zigzag, causal=causal, kpm=kpm, rope_base=rope,
                                    flags=bosa.ATTN_NO_TILE_SKIP)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), o2.cpu()) and torch.equal(lse.cpu(), l2.cpu()), f"rank {rank}: NO_TILE_SKIP"


@pytest.mark.parametrize("zigzag,causal,dtype", [(True, True, torch.bfloat16), (False, False, torch.bfloat16),
                                                 (False, True, torch.float32)])
def test_ring_share_with_a_fully_padded_row(zigzag, causal, dtype):
    """attn_ring_fwd where every key of batch row 1 is padded: each of that
    row's sub-calls has no live tile (the chained kernel's workgroups of that
    row end with an empty state), so its rows come out as the merge identity,
    out = 0 and lse = -inf; row 0 (random holes) still matches the oracle,
    every rank."""
    P, B, H, T, d = 4, 2, 2, 1024, 128
    kpm = workloads.random_mask((B, T), 9600 + int(zigzag), 0.2)
    kpm[1, :] = 1
    for rank in range(P):
        qpos = oracle.local_query_positions(T, P, rank, zigzag)
        seed = 9610 + 10 * rank + int(zigzag)
        q = rnd((B, T // P, H, d), seed, dtype)
        k = rnd((B, T, H, d), seed + 1, dtype)
        v = rnd((B, T, H, d), seed + 2, dtype)
        note(f"ring fully padded row: zigzag={zigzag} causal={causal} {dtype} rank={rank}")
        out, lse = bosa.attn_ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P=P, rank=rank, zigzag=zigzag, causal=causal,
                                      kpm=kpm.to(DEV), rope_base=10000.0)
        torch.cuda.synchronize()
        ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=causal, kpm=kpm.numpy(),
                             rope_base=10000.0, dtype=dt_name(q))
        assert np.all(np.isneginf(rl[1])) and not np.any(ro[1])
        compare(out.cpu(), lse.cpu(), ro, rl, dt_name(q), f"rank{rank}")


@pytest.mark.parametrize("zigzag", [True, False])
def test_ring_share_batch_rows_with_different_padding(zigzag):
    """attn_ring_fwd with B*H a multiple of 8 and batch rows padded to
    different lengths (the chained kernel then spreads the (batch row, head)
    pairs over the XCDs round-robin): B = 2, H = 4, P = 4, every rank,
    against the oracle."""
    P, B, H, T, d = 4, 2, 4, 1024, 128
    kpm = torch.zeros((B, T), dtype=torch.uint8)
    kpm[0, 900:] = 1
    kpm[1, 333:] = 1
    for rank in range(P):
        qpos = oracle.local_query_positions(T, P, rank, zigzag)
        seed = 9900 + 10 * rank + int(zigzag)
        q = rnd((B, T // P, H, d), seed, torch.bfloat16)
        k = rnd((B, T, H, d), seed + 1, torch.bfloat16)
        v = rnd((B, T, H, d), seed + 2, torch.bfloat16)
        note(f"ring share, uneven padding: zigzag={zigzag} rank={rank}")
        out, lse = bosa.attn_ring_fwd(q.to(DEV), k.to(DEV), v.to(DEV), P=P, rank=rank, zigzag=zigzag, causal=True,
                                      kpm=kpm.to(DEV), rope_base=10000.0)
        torch.cuda.synchronize()
        ro, rl = oracle.sdpa(np64(q), np64(k), np64(v), qpos, np.arange(T), causal=True, kpm=kpm.numpy(),
                             rope_base=10000.0, dtype="bf16")
        compare(out.cpu(), lse.cpu(), ro, rl, "bf16", f"rank{rank}")
