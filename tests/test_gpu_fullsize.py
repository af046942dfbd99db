"""Parity at the full workload sizes, in the launch configuration bench.py
times (attn_ring_fwd for the ring shares, one attn_fwd call otherwise).

The oracle cannot afford every row at these sizes, so it recomputes sampled
query rows (chunk starts and ends, tile boundaries, random rows) for sampled
heads, each against every key at its absolute position.  Properties that hold
at any size are checked on every row: finite outputs, no empty rows, and
rows summing to one (V = 1) for the largest share.
"""
import numpy as np
import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle
import workloads
from gpu_helpers import DEV, compare, note, np64

pytestmark = pytest.mark.gpu


def _sample_rows(n, chunk, rng, extra=24):
    rows = set()
    for c0 in range(0, n, chunk):
        rows.update([c0, c0 + 1, c0 + 127, c0 + 128, c0 + chunk - 1])
    rows.update(rng.choice(n, size=extra, replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n))


def _ring_inputs(w):
    P, rank = w.ring_P, w.ring_rank
    qpos = oracle.local_query_positions(w.T, P, rank, w.zigzag)
    chunks = [int(qpos[0] // w.chunk)]
    if w.zigzag:
        chunks.append(int(qpos[-1] // w.chunk))
    q = workloads.draw_tokens(w, 0, chunks)
    k = workloads.draw_tokens(w, 1, range(w.n_chunks))
    v = workloads.draw_tokens(w, 2, range(w.n_chunks))
    return q, k, v, qpos


@pytest.mark.parametrize("wi,rank", [(2, None), (4, None), (4, 7)])
def test_ring_share_full_size_sampled(wi, rank):
    w = workloads.WORKLOADS[wi]
    if rank is not None:
        w = workloads.Workload(**{**w.__dict__, "ring_rank": rank})
    note(f"{w.name} rank={w.ring_rank}: drawing inputs")
    q, k, v, qpos = _ring_inputs(w)
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    note("  running attn_ring_fwd")
    out, lse = bosa.attn_ring_fwd(dq, dk, dv, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag, causal=w.causal,
                                  rope_base=w.rope_base)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(wi * 10 + w.ring_rank)
    rows = _sample_rows(q.shape[1], q.shape[1] // (2 if w.zigzag else 1), rng)
    heads = sorted({0, w.H // 2 - 1, w.H - 1, int(rng.integers(w.H))})
    oc, lc = out.cpu(), lse.cpu()
    for h in heads:
        note(f"  oracle: {len(rows)} rows of head {h}")
        ro, rl = oracle.sdpa(np64(q[:, rows, h:h + 1]), np64(k[:, :, h:h + 1]), np64(v[:, :, h:h + 1]), qpos[rows],
                             np.arange(w.T), causal=w.causal, rope_base=w.rope_base, dtype="bf16")
        compare(oc[:, rows, h:h + 1], lc[:, h:h + 1, rows], ro, rl, "bf16", f"head{h}")
    if wi == 4 and rank is None:
        # the share's first rows see one to four keys (global positions 0-3
        # under causal order): there a rounding step of the rotated operands
        # moves lse most, so every head of them is checked and reported
        first = np.arange(4)
        el_first = eo_first = 0.0
        for h in range(w.H):
            ro, rl = oracle.sdpa(np64(q[:, first, h:h + 1]), np64(k[:, :4, h:h + 1]), np64(v[:, :4, h:h + 1]),
                                 qpos[first], np.arange(4), causal=True, rope_base=w.rope_base, dtype="bf16")
            eo_first = max(eo_first, float(np.abs(np64(oc[:, first, h:h + 1]) - ro).max()))
            el_first = max(el_first, float(np.abs(np64(lc[:, h:h + 1, first]) - rl).max()))
        note(f"  rows 0-3 (1-4 keys), all {w.H} heads: max|dout|={eo_first:.3e} max|dlse|={el_first:.3e}")
        assert eo_first <= 2e-2 and el_first <= 1e-3
        # rows sum to one: V = 1 gives out = 1 on every row and head
        ones = torch.ones_like(dv)
        o1, _ = bosa.attn_ring_fwd(dq, dk, ones, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag, causal=w.causal,
                                   rope_base=w.rope_base)
        torch.cuda.synchronize()
        err = float((o1.float() - 1).abs().max())
        note(f"  V=1 max|out-1| = {err:.3e}")
        assert err <= 2e-2


def test_encoder_full_size_sampled():
    w = workloads.WORKLOADS[3]
    note(f"{w.name}: drawing inputs")
    q, k, v = (workloads.draw_tokens(w, t, range(w.n_chunks)) for t in (0, 1, 2))
    kpm = workloads.key_padding_mask(w)
    out, lse = bosa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), kpm=kpm.to(DEV), causal=False)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(3)
    rows = _sample_rows(w.T, 4096, rng)
    oc, lc = out.cpu(), lse.cpu()
    for b in range(w.B):
        for h in sorted({0, w.H - 1, int(rng.integers(w.H))}):
            note(f"  oracle: batch {b} head {h} ({len(rows)} rows, valid keys {int((kpm[b] == 0).sum())})")
            ro, rl = oracle.attention(np64(q[b:b + 1, rows, h:h + 1]), np64(k[b:b + 1, :, h:h + 1]),
                                      np64(v[b:b + 1, :, h:h + 1]), kpm=kpm[b:b + 1].numpy(), dtype="bf16")
            # rows are a subset, positions do not matter without causal order or RoPE
            compare(oc[b:b + 1, rows, h:h + 1], lc[b:b + 1, h:h + 1, rows], ro, rl, "bf16", f"b{b}h{h}")


def test_head_parallel_share_full_size_sampled():
    """One rank's share under the head-parallel (Ulysses) layout of the 128K
    sequence: 4 of 32 heads over all 131072 tokens, causal, RoPE, in one
    attn_fwd call (the call that rank makes after its all-to-all).  Sampled
    rows of every head against the oracle; every row finite."""
    w = workloads.WORKLOADS[6]
    note(f"{w.name}: drawing inputs")
    q, k, v = (workloads.draw_tokens(w, t, range(w.n_chunks)) for t in (0, 1, 2))
    out, lse = bosa.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, rope_base=w.rope_base)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(6)
    rows = _sample_rows(w.T, w.chunk, rng, extra=16)
    oc, lc = out.cpu(), lse.cpu()
    for h in range(w.H):
        nk = int(rows.max()) + 1
        note(f"  oracle: {len(rows)} rows of head {h}")
        ro, rl = oracle.sdpa(np64(q[:, rows, h:h + 1]), np64(k[:, :nk, h:h + 1]), np64(v[:, :nk, h:h + 1]), rows,
                             np.arange(nk), causal=True, rope_base=w.rope_base, dtype="bf16")
        compare(oc[:, rows, h:h + 1], lc[:, h:h + 1, rows], ro, rl, "bf16", f"head{h}")


def test_ring_backward_full_size_sampled():
    """The backward of the 128K zigzag share (rank 0) in the launch
    configuration `bench.py --pass bwd` times: attn_ring_bwd (bf16 gradients)
    after attn_ring_fwd.  Every gradient is finite; dq of sampled rows of
    sampled heads matches the oracle (dq of a row depends on that row alone);
    and dv obeys the exact identity sum_j dv_j = sum_i dout_i per (head,
    coordinate), since every row's probabilities sum to one.  The identity is
    checked within the rounding it allows: bf16 probabilities and bf16
    outputs, at most 2^-9 relative each (doubled for margin).  dk and dv of
    sampled key rows of every chunk (chunk 0, which two sub-calls touch, goes
    through the float32 finalize pass; the other chunks get their final bf16
    gradients from the dK/dV kernel) on one head match the oracle's block
    gradients, built from the oracle's own out and lse of all 16384 local
    rows."""
    w = workloads.WORKLOADS[4]
    note(f"{w.name}: drawing inputs")
    q, k, v, qpos = _ring_inputs(w)
    chunks = [int(qpos[0] // w.chunk), int(qpos[-1] // w.chunk)]
    dout = workloads.draw_tokens(w, 4, chunks)
    dq_, dk_, dv_ = q.to(DEV), k.to(DEV), v.to(DEV)
    note("  running attn_ring_fwd + attn_ring_bwd")
    out, lse = bosa.attn_ring_fwd(dq_, dk_, dv_, P=w.ring_P, rank=w.ring_rank, zigzag=w.zigzag, causal=w.causal,
                                  rope_base=w.rope_base)
    gq, gk, gv = bosa.attn_ring_bwd(dq_, dk_, dv_, out, dout.to(DEV), lse, P=w.ring_P, rank=w.ring_rank,
                                    zigzag=w.zigzag, causal=w.causal, rope_base=w.rope_base)
    torch.cuda.synchronize()
    for name, g in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert torch.isfinite(g.float()).all(), f"{name}: non-finite gradient"
    rng_k = np.random.default_rng(45)
    hk = int(rng_k.integers(w.H))
    krows = _sample_rows(w.T, w.chunk, rng_k, extra=16)
    krows = np.array(sorted(set(krows.tolist()) | {c0 + 4095 for c0 in range(0, w.T, w.chunk)}))
    kidx = torch.from_numpy(krows).to(DEV)
    gk_s = gk[:, kidx, hk:hk + 1].cpu()
    gv_s = gv[:, kidx, hk:hk + 1].cpu()
    gq, gv = gq.cpu(), gv.cpu()
    del out, lse, gk, dq_, dk_, dv_
    # dq of sampled rows
    rng = np.random.default_rng(44)
    rows = _sample_rows(q.shape[1], q.shape[1] // 2, rng, extra=16)
    for h in sorted({0, w.H - 1, int(rng.integers(w.H))}):
        nk = int(qpos[rows].max()) + 1
        note(f"  oracle: dq of {len(rows)} rows of head {h}")
        rq, _, _ = oracle.sdpa_backward(np64(q[:, rows, h:h + 1]), np64(k[:, :nk, h:h + 1]),
                                        np64(v[:, :nk, h:h + 1]), np64(dout[:, rows, h:h + 1]), qpos[rows],
                                        np.arange(nk), causal=True, rope_base=w.rope_base, dtype="bf16")
        g = np64(gq[:, rows, h:h + 1])
        e = float(np.abs(g - rq).max()) / float(np.abs(rq).max())
        note(f"  head {h} dq: max|err|/max|ref| = {e:.3e}")
        assert e <= 2e-2, f"dq head {h}: relative error {e}"
    # sum_j dv_j = sum_i dout_i for every (head, coordinate)
    sv = np.zeros((w.H, w.d))
    av = np.zeros((w.H, w.d))
    for t0 in range(0, w.T, 8192):
        blk = np64(gv[0, t0:t0 + 8192])
        sv += blk.sum(axis=0)
        av += np.abs(blk).sum(axis=0)
    so = np64(dout[0]).sum(axis=0)
    ao = np.abs(np64(dout[0])).sum(axis=0)
    err = np.abs(sv - so)
    bound = 2.0 * 2.0 ** -9 * (av + ao)
    note(f"  sum dv - sum dout: max {err.max():.3e}, worst fraction of its bound {(err / bound).max():.3f}")
    assert np.all(err <= bound)
    # dk, dv of sampled key rows of head hk: the oracle's out and lse of every
    # local row (rows are independent in the forward), then its block gradients
    Tl = q.shape[1]
    qh, kh, vh, gh = (np64(x[:, :, hk:hk + 1]) for x in (q, k, v, dout))
    o_ref = np.zeros((1, Tl, 1, w.d))
    l_ref = np.zeros((1, 1, Tl))
    note(f"  oracle: out and lse of all {Tl} local rows of head {hk}")
    for r0 in range(0, Tl, 512):
        rr = np.arange(r0, min(r0 + 512, Tl))
        nk = int(qpos[rr].max()) + 1
        o_ref[:, rr], l_ref[:, :, rr] = oracle.sdpa(qh[:, rr], kh[:, :nk], vh[:, :nk], qpos[rr], np.arange(nk),
                                                    causal=True, rope_base=w.rope_base, dtype="bf16")
    note(f"  oracle: dk, dv of {len(krows)} key rows of head {hk}")
    rk, rv = oracle.key_block_gradients(qh, kh, vh, gh, o_ref, l_ref, qpos, np.arange(w.T), krows, causal=True,
                                        rope_base=w.rope_base, dtype="bf16")
    for name, got, ref in (("dk", gk_s, rk), ("dv", gv_s, rv)):
        e = float(np.abs(np64(got) - ref).max()) / float(np.abs(ref).max())
        note(f"  head {hk} {name} of sampled keys: max|err|/max|ref| = {e:.3e}")
        assert e <= 2e-2, f"{name} head {hk}: relative error {e}"


def test_head_parallel_backward_full_size_sampled():
    """The backward of the head-parallel share (4 heads x 131072 tokens,
    causal, RoPE) in the configuration `bench.py --workload 6 --pass bwd`
    times: one attn_bwd call (bf16 gradients, so every key block's dk and dv
    are written as final bf16 by the dK/dV kernel).  Every gradient is
    finite; dq of sampled rows on two heads matches the oracle; dk and dv of
    sampled keys of the last chunk on one head match the oracle's block
    gradients, built from the oracle's own out and lse of the rows that see
    those keys (causal order: the last 8192 rows)."""
    w = workloads.WORKLOADS[6]
    note(f"{w.name}: drawing inputs")
    q, k, v = (workloads.draw_tokens(w, t, range(w.n_chunks)) for t in (0, 1, 2))
    dout = workloads.draw_tokens(w, 4, range(w.n_chunks))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    note("  running attn_fwd + attn_bwd")
    out, lse = bosa.attn_fwd(qd, kd, vd, causal=True, rope_base=w.rope_base)
    gq, gk, gv = bosa.attn_bwd(qd, kd, vd, out, dout.to(DEV), lse, causal=True, rope_base=w.rope_base)
    torch.cuda.synchronize()
    for name, g in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert torch.isfinite(g.float()).all(), f"{name}: non-finite gradient"
    gq, gk, gv = gq.cpu(), gk.cpu(), gv.cpu()
    del out, lse, qd, kd, vd
    pos = np.arange(w.T)
    rng = np.random.default_rng(66)
    rows = _sample_rows(w.T, w.chunk, rng, extra=8)
    for h in (0, w.H - 1):
        nk = int(rows.max()) + 1
        note(f"  oracle: dq of {len(rows)} rows of head {h}")
        rq, _, _ = oracle.sdpa_backward(np64(q[:, rows, h:h + 1]), np64(k[:, :nk, h:h + 1]), np64(v[:, :nk, h:h + 1]),
                                        np64(dout[:, rows, h:h + 1]), rows, np.arange(nk), causal=True,
                                        rope_base=w.rope_base, dtype="bf16")
        e = float(np.abs(np64(gq[:, rows, h:h + 1]) - rq).max()) / float(np.abs(rq).max())
        note(f"  head {h} dq: max|err|/max|ref| = {e:.3e}")
        assert e <= 2e-2, f"dq head {h}: relative error {e}"
    # dk, dv of sampled keys of the last chunk: only rows r0.. see them
    r0 = w.T - w.chunk
    krows = np.array(sorted({r0, r0 + 1, r0 + 63, r0 + 64, r0 + 4095, w.T - 2, w.T - 1}
                            | set((r0 + rng.choice(w.chunk, size=24, replace=False)).tolist())))
    h = int(rng.integers(w.H))
    seen = np.arange(r0, w.T)
    qh, kh, vh, gh = np64(q[:, seen, h:h + 1]), np64(k[:, :, h:h + 1]), np64(v[:, :, h:h + 1]), np64(dout[:, seen, h:h + 1])
    o_ref = np.zeros((1, len(seen), 1, w.d))
    l_ref = np.zeros((1, 1, len(seen)))
    note(f"  oracle: out and lse of rows {r0}..{w.T - 1} of head {h}")
    for b0 in range(0, len(seen), 512):
        rr = np.arange(b0, min(b0 + 512, len(seen)))
        nk = int(seen[rr].max()) + 1
        o_ref[:, rr], l_ref[:, :, rr] = oracle.sdpa(qh[:, rr], kh[:, :nk], vh[:, :nk], seen[rr], np.arange(nk),
                                                    causal=True, rope_base=w.rope_base, dtype="bf16")
    note(f"  oracle: dk, dv of {len(krows)} key rows of head {h}")
    rk, rv = oracle.key_block_gradients(qh, kh, vh, gh, o_ref, l_ref, seen, pos, krows, causal=True,
                                        rope_base=w.rope_base, dtype="bf16")
    for name, got, ref in (("dk", gk[:, krows, h:h + 1], rk), ("dv", gv[:, krows, h:h + 1], rv)):
        e = float(np.abs(np64(got) - ref).max()) / float(np.abs(ref).max())
        note(f"  head {h} {name} of sampled keys: max|err|/max|ref| = {e:.3e}")
        assert e <= 2e-2, f"{name} head {h}: relative error {e}"
