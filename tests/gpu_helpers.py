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
