"""Shared helpers of the GPU parity tests: run the library through its C ABI
and compare against the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import blockwise_online_softmax_attn_amd as bosa
import oracle

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}   # (out max-abs, lse max-abs)
DEV = "cuda:0"


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dt_name(t: torch.Tensor) -> str:
    return "f32" if t.dtype == torch.float32 else "bf16"


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def gpu_fwd(q, k, v, **kw):
    """attn_fwd on device copies of the CPU tensors; returns CPU tensors."""
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    for name in ("kpm", "attn_mask"):
        if kw.get(name) is not None:
            kw[name] = kw[name].to(DEV)
    out, lse = bosa.attn_fwd(dq, dk, dv, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def ref_fwd(q, k, v, *, q_off=0, kv_off=0, causal=False, kpm=None, attn_mask=None, rope_base=0.0):
    return oracle.attention(np64(q), np64(k), np64(v), q_off=q_off, kv_off=kv_off, causal=causal,
                            kpm=None if kpm is None else kpm.numpy(),
                            attn_mask=None if attn_mask is None else attn_mask.numpy(),
                            rope_base=rope_base, dtype=dt_name(q))


def compare(out, lse, ref_out, ref_lse, dtype: str, what: str = ""):
    """Max-abs parity (lse compared where finite; -inf must match exactly),
    plus the log10 L2 error per row that is reported alongside."""
    tol_o, tol_l = TOL[dtype]
    o = np64(out)
    l = np64(lse)
    assert o.shape == ref_out.shape and l.shape == ref_lse.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: empty-row pattern differs"
    assert np.all(l[~fin] == -np.inf)
    if dtype == "f32" and fin.any():
        # a float32 lse is itself rounded to half a unit in the last place of
        # its magnitude; where distance penalties make |lse| large (ALiBi),
        # 1e-5 falls below a few such units, so 4 of them are allowed.  The
        # scores behind it are float32 numbers of that magnitude too: half a
        # unit of |score| in the exponent is a relative error of P, so out
        # (a P-weighted mean of unit-variance v rows) gets the same 4 units.
        unit = float(np.spacing(np.float32(np.abs(ref_lse[fin]).max())))
        tol_l = max(tol_l, 4.0 * unit)
        tol_o = max(tol_o, 4.0 * unit)
    eo = float(np.abs(o - ref_out).max()) if o.size else 0.0
    el = float(np.abs(l[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    row_err = np.sqrt(((o - ref_out) ** 2).sum(-1)) + 1e-300
    note(f"  {what}: max|dout|={eo:.3e} (tol {tol_o}) max|dlse|={el:.3e} (tol {tol_l}) "
         f"log10 L2 row err max={np.log10(row_err.max()):.2f} mean={np.log10(row_err).mean():.2f}")
    assert eo <= tol_o, f"{what}: out error {eo} > {tol_o}"
    assert el <= tol_l, f"{what}: lse error {el} > {tol_l}"
    return eo, el


CHAIN_MAX = 16     # sub-calls per launch of the chained ring executor
CHAIN_ROWS = 256   # query rows per workgroup of that launch


def ring_chains(plan, B, H, causal, n_cu):
    """The launches of the chained ring executor (bf16, no window or ALiBi):
    per query block, its sub-calls in plan order, at most CHAIN_MAX to a
    launch, and a launch also ends after a sub-call that causal order cuts
    through the query block when the launch has more workgroups than the
    device has CUs.  Returns lists of plan entries."""
    chains = []
    for ph in (0, 1):
        sub = [e for e in plan if (0 if e.q_row0 == 0 else 1) == ph]
        cur = []
        for e in sub:
            cur.append(e)
            wgs = B * H * -(-e.q_rows // CHAIN_ROWS)
            cut = causal and wgs > n_cu and e.kv_pos0 + e.kv_rows - 1 > e.q_pos0
            if len(cur) == CHAIN_MAX or cut:
                chains.append(cur)
                cur = []
        if cur:
            chains.append(cur)
    return chains


def chained_ring_reference(q, k, v, kpm, P, rank, zigzag, causal, rope):
    """What attn_ring_fwd's chained executor computes, rebuilt from plain
    attn_fwd calls: each launch's blocks act as one key sequence, so each
    launch becomes one attn_fwd over its blocks' keys concatenated in ring
    order, each block padded to whole 64-key tiles with excluded zero keys
    (as the executor's tiles are), with causal order as an attention mask over
    absolute positions and the rotations applied beforehand by rope_apply;
    launches after a query block's first merge into its float32 partial, then
    one cast.  Equal to the executor bit for bit (the tile sequence and every
    tile's arithmetic are the same; fully masked tiles that one side skips
    change no bit)."""
    B, Tl, H, d = q.shape
    T = k.shape[1]
    plan = bosa.attn_ring_plan(T, P, rank, zigzag, causal)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    kpos = torch.arange(T, device=DEV)
    qpos = torch.from_numpy(oracle.local_query_positions(T, P, rank, zigzag)).to(DEV)
    qr, kr = q.clone(), k.clone()
    if rope > 0:
        bosa.rope_apply(qr, qpos, rope)
        bosa.rope_apply(kr, kpos, rope)
    acc = torch.zeros((B, Tl, H, d), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, Tl), float("-inf"), device=DEV)
    parts = {}
    for chain in ring_chains(plan, B, H, causal, n_cu):
        r0, nr = chain[0].q_row0, chain[0].q_rows
        widths = [-(-e.kv_rows // 64) * 64 for e in chain]
        n = sum(widths)
        kc = torch.zeros((B, n, H, d), dtype=k.dtype, device=DEV)
        vc = torch.zeros((B, n, H, d), dtype=v.dtype, device=DEV)
        am = torch.ones((nr, n), dtype=torch.uint8, device=DEV)   # padding keys: excluded
        kpc = None if kpm is None else torch.ones((B, n), dtype=torch.uint8, device=DEV)
        c0 = 0
        for e, wdt in zip(chain, widths):
            sl = slice(e.kv_pos0, e.kv_pos0 + e.kv_rows)
            kc[:, c0:c0 + e.kv_rows] = kr[:, sl]
            vc[:, c0:c0 + e.kv_rows] = v[:, sl]
            keys = kpos[sl]
            if causal:
                am[:, c0:c0 + e.kv_rows] = (keys[None, :] > qpos[r0:r0 + nr, None]).to(torch.uint8)
            else:
                am[:, c0:c0 + e.kv_rows] = 0
            if kpm is not None:
                kpc[:, c0:c0 + e.kv_rows] = kpm[:, sl]
            c0 += wdt
        if r0 not in parts:
            parts[r0] = (torch.empty((B, nr, H, d), dtype=torch.float32, device=DEV),
                         torch.empty((B, H, nr), dtype=torch.float32, device=DEV))
        a, la = parts[r0]
        flags = bosa.ATTN_OUT_F32 | (bosa.ATTN_ACCUMULATE if chain[0].accumulate else 0)
        bosa.attn_fwd(qr[:, r0:r0 + nr].contiguous(), kc, vc, a, la, causal=False, kpm=kpc,
                      attn_mask=am.contiguous(), flags=flags)
    for r0, (a, la) in parts.items():
        acc[:, r0:r0 + a.shape[1]] = a
        lse[:, :, r0:r0 + a.shape[1]] = la
    out = torch.empty((B, Tl, H, d), dtype=torch.bfloat16, device=DEV)
    bosa.attn_cast(acc, out)
    torch.cuda.synchronize()
    return out, lse
