"""Blockwise online-softmax attention (forward and backward) for AMD Instinct
MI355X (gfx950).

Python binding of libattn.so (C ABI in include/attn.h).  These functions only
marshal arguments: they check tensor placement, shapes and dtypes, allocate
outputs the caller did not pass, and hand raw device pointers and the current
HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

import torch

from ._lib import (  # noqa: F401
    ATTN_ACCUMULATE,
    ATTN_BF16,
    ATTN_F32,
    ATTN_NO_TILE_SKIP,
    ATTN_OUT_F32,
    AttnError,
    EXPORTS,
    LIB_PATH,
    RingCall,
    Variant,
    check,
    load,
)

_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DTYPES[t.dtype]


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


def _variant(window, alibi_slopes, H: int):
    """attn_variant for a (left, right) window and [H] float32 slopes, or None."""
    if window is None and alibi_slopes is None:
        return None, None
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    if alibi_slopes is not None and (alibi_slopes.shape != (H,) or alibi_slopes.dtype != torch.float32):
        raise ValueError("alibi_slopes must be float32 of shape (H,)")
    v = Variant(wl, wr, _dev(alibi_slopes, "alibi_slopes", torch.float32))
    return ctypes.byref(v), v


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, *, q_off: int = 0, kv_off: int = 0, causal: bool = False,
             kpm: Optional[torch.Tensor] = None, attn_mask: Optional[torch.Tensor] = None,
             rope_base: float = 0.0, flags: int = 0, window=None, alibi_slopes: Optional[torch.Tensor] = None,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """out, lse = attention over one key/value block (see attn_fwd in attn.h).

    q (B, Tq, H, d), k/v (B, Tkv, H, d); kpm (B, Tkv) and attn_mask (Tq, Tkv)
    are uint8 with nonzero = excluded.  out is allocated in q's dtype, or
    float32 with ATTN_OUT_F32; lse (B, H, Tq) float32.  window = (left,
    right) (-1 = no limit) and alibi_slopes (H,) float32 select attn_fwd_ex."""
    load()
    B, Tq, H, d = q.shape
    Tkv = k.shape[1]
    if k.shape != (B, Tkv, H, d) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    code = _dtype_code(q)
    out_dtype = torch.float32 if (flags & ATTN_OUT_F32) else q.dtype
    if out is None:
        if flags & ATTN_ACCUMULATE:
            raise ValueError("ATTN_ACCUMULATE needs the partial out and lse to merge into")
        out = torch.empty((B, Tq, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    if out.shape != (B, Tq, H, d) or lse.shape != (B, H, Tq):
        raise ValueError("out/lse shape mismatch")
    if kpm is not None and (kpm.shape != (B, Tkv) or kpm.dtype != torch.uint8):
        raise ValueError("kpm must be uint8 (B, Tkv)")
    if attn_mask is not None and (attn_mask.shape != (Tq, Tkv) or attn_mask.dtype != torch.uint8):
        raise ValueError("attn_mask must be uint8 (Tq, Tkv)")
    args = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out", out_dtype), _dev(lse, "lse", torch.float32),
            B, H, Tq, Tkv, d, int(q_off), int(kv_off), 1 if causal else 0, _dev(kpm, "kpm"),
            _dev(attn_mask, "attn_mask"), float(rope_base), code, int(flags))
    var, _keep = _variant(window, alibi_slopes, H)
    if var is None:
        rc = load().attn_fwd(*args, _stream(stream))
    else:
        rc = load().attn_fwd_ex(*args, var, _stream(stream))
    check(rc)
    return out, lse


def attn_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cache_len: torch.Tensor, *, rope_base: float = 0.0, stream=None) -> None:
    """Append one token per row to a static cache (see attn_kv_append in attn.h):
    k_new, v_new (B, H, d); caches (B, Tcap, H, d); cache_len int32 (B,) on the
    device, advanced by one for every row that had room."""
    load()
    B, Tcap, H, d = k_cache.shape
    if v_cache.shape != k_cache.shape or k_new.shape != (B, H, d) or v_new.shape != (B, H, d):
        raise ValueError("cache / new-token shape mismatch")
    if cache_len.shape != (B,):
        raise ValueError("cache_len must have shape (B,)")
    for t in (k_new, v_new, v_cache):
        if t.dtype != k_cache.dtype:
            raise TypeError("k_new, v_new and the caches must share a dtype")
    rc = load().attn_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
                               _dev(v_cache, "v_cache"), _dev(cache_len, "cache_len", torch.int32), B, H, Tcap, d,
                               float(rope_base), _dtype_code(k_cache), _stream(stream))
    check(rc)


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_len: torch.Tensor,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *, rope_base: float = 0.0,
                window_left: int = -1, alibi_slopes: Optional[torch.Tensor] = None, flags: int = 0,
                noalloc: bool = False, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """out (B, H, d), lse (B, H) of each row's newest query over its cache
    (see attn_decode in attn.h).  noalloc selects attn_decode_noalloc (the
    library allocates nothing; pass out and lse to allocate nothing here
    either)."""
    load()
    B, Tcap, H, d = k_cache.shape
    if v_cache.shape != k_cache.shape or q.shape != (B, H, d):
        raise ValueError("q / cache shape mismatch")
    if cache_len.shape != (B,):
        raise ValueError("cache_len must have shape (B,)")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    out_dtype = torch.float32 if (flags & ATTN_OUT_F32) else q.dtype
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, d) or lse.shape != (B, H):
        raise ValueError("out/lse shape mismatch")
    var, _keep = _variant((window_left, -1) if window_left >= 0 else None, alibi_slopes, H)
    fn = load().attn_decode_noalloc if noalloc else load().attn_decode
    rc = fn(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                            _dev(cache_len, "cache_len", torch.int32), _dev(out, "out", out_dtype),
                            _dev(lse, "lse", torch.float32), B, H, Tcap, d, float(rope_base), _dtype_code(q),
                            int(flags), var, _stream(stream))
    check(rc)
    return out, lse


def attn_merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor, lse_b: torch.Tensor,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(out_a, lse_a) <- merge with (out_b, lse_b), in place; out_a float32."""
    load()
    B, Tq, H, d = out_a.shape
    if out_b.shape != out_a.shape or lse_a.shape != (B, H, Tq) or lse_b.shape != (B, H, Tq):
        raise ValueError("merge shape mismatch")
    rc = load().attn_merge(_dev(out_a, "out_a", torch.float32), _dev(lse_a, "lse_a", torch.float32),
                           _dev(out_b, "out_b"), _dev(lse_b, "lse_b", torch.float32), B, H, Tq, d,
                           _dtype_code(out_b), _stream(stream))
    check(rc)
    return out_a, lse_a


def rope_apply(x: torch.Tensor, pos: torch.Tensor, base: float, stream=None) -> torch.Tensor:
    """Rotary embedding of x (B, T, H, d) in place; pos int64 (T,) on the device."""
    load()
    B, T, H, d = x.shape
    if pos.shape != (T,):
        raise ValueError("pos must have shape (T,)")
    rc = load().rope_apply(_dev(x, "x"), _dev(pos, "pos", torch.int64), float(base), B, T, H, d,
                           _dtype_code(x), _stream(stream))
    check(rc)
    return x


def attn_cast(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    load()
    if src.numel() != dst.numel():
        raise ValueError("size mismatch")
    rc = load().attn_cast(_dev(src, "src", torch.float32), _dev(dst, "dst"), src.numel(), _dtype_code(dst),
                          _stream(stream))
    check(rc)
    return dst


def attn_ring_plan(T: int, P: int, rank: int, zigzag: bool, causal: bool) -> List[RingCall]:
    """The sub-calls of one rank's ring share, in issue order (host only)."""
    lib = load()
    n = lib.attn_ring_plan(T, P, rank, int(zigzag), int(causal), None, 0)
    if n < 0:
        check(-n)
    buf = (RingCall * max(n, 1))()
    lib.attn_ring_plan(T, P, rank, int(zigzag), int(causal), buf, n)
    return [buf[i] for i in range(n)]


def attn_ring_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, P: int, rank: int, zigzag: bool,
                  causal: bool = True, kpm: Optional[torch.Tensor] = None, rope_base: float = 0.0, flags: int = 0,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  acc: Optional[torch.Tensor] = None, window=None, alibi_slopes: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One rank's ring-attention share: local q (B, T/P, H, d) against the
    full k, v (B, T, H, d) in ring order, merged into (out, lse).  window /
    alibi_slopes select attn_ring_fwd_ex."""
    load()
    B, T, H, d = k.shape
    Tl = q.shape[1]
    if q.shape != (B, T // P, H, d) or Tl * P != T or v.shape != k.shape:
        raise ValueError("ring shapes: q (B, T/P, H, d), k = v (B, T, H, d)")
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Tl), dtype=torch.float32, device=q.device)
    if acc is None:
        acc = out if q.dtype == torch.float32 else torch.empty(q.shape, dtype=torch.float32, device=q.device)
    args = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out", q.dtype), _dev(lse, "lse", torch.float32),
            _dev(acc, "acc", torch.float32), B, H, T, d, P, rank, int(zigzag), int(causal), _dev(kpm, "kpm"),
            float(rope_base), code, int(flags))
    var, _keep = _variant(window, alibi_slopes, H)
    if var is None:
        rc = load().attn_ring_fwd(*args, _stream(stream))
    else:
        rc = load().attn_ring_fwd_ex(*args, var, _stream(stream))
    check(rc)
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, *, q_off: int = 0, kv_off: int = 0, causal: bool = False,
             kpm: Optional[torch.Tensor] = None, attn_mask: Optional[torch.Tensor] = None, rope_base: float = 0.0,
             flags: int = 0, window=None, alibi_slopes: Optional[torch.Tensor] = None,
             stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dq, dk, dv of sum(dout * out) for the attn_fwd call with the same
    arguments (see attn_bwd in attn.h).  bf16 inputs; gradients bf16, or
    float32 with ATTN_OUT_F32 (ATTN_ACCUMULATE adds into dq, dk, dv).
    window / alibi_slopes as for attn_fwd select attn_bwd_ex."""
    load()
    B, Tq, H, d = q.shape
    Tkv = k.shape[1]
    if k.shape != (B, Tkv, H, d) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse.shape != (B, H, Tq):
        raise ValueError("lse must be (B, H, Tq)")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    gdt = torch.float32 if (flags & ATTN_OUT_F32) else torch.bfloat16
    if flags & ATTN_ACCUMULATE and (dq is None or dk is None or dv is None):
        raise ValueError("ATTN_ACCUMULATE needs dq, dk and dv to add into")
    dq = torch.empty(q.shape, dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=gdt, device=q.device) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("gradient shape mismatch")
    if kpm is not None and (kpm.shape != (B, Tkv) or kpm.dtype != torch.uint8):
        raise ValueError("kpm must be uint8 (B, Tkv)")
    if attn_mask is not None and (attn_mask.shape != (Tq, Tkv) or attn_mask.dtype != torch.uint8):
        raise ValueError("attn_mask must be uint8 (Tq, Tkv)")
    args = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(dout, "dout"),
            _dev(lse, "lse", torch.float32), _dev(dq, "dq", gdt), _dev(dk, "dk", gdt), _dev(dv, "dv", gdt),
            B, H, Tq, Tkv, d, int(q_off), int(kv_off), 1 if causal else 0, _dev(kpm, "kpm"),
            _dev(attn_mask, "attn_mask"), float(rope_base), ATTN_BF16, int(flags))
    var, _keep = _variant(window, alibi_slopes, H)
    if var is None:
        rc = load().attn_bwd(*args, _stream(stream))
    else:
        rc = load().attn_bwd_ex(*args, var, _stream(stream))
    check(rc)
    return dq, dk, dv


def attn_ring_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, *, P: int, rank: int, zigzag: bool, causal: bool = True,
                  kpm: Optional[torch.Tensor] = None, rope_base: float = 0.0, flags: int = 0,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, window=None, alibi_slopes: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of one rank's ring share: local q, out, dout (B, T/P, H, d),
    full k, v (B, T, H, d), lse from attn_ring_fwd.  Returns dq (local) and
    this rank's contributions dk, dv (full length)."""
    load()
    B, T, H, d = k.shape
    Tl = q.shape[1]
    if q.shape != (B, T // P, H, d) or Tl * P != T or v.shape != k.shape:
        raise ValueError("ring shapes: q (B, T/P, H, d), k = v (B, T, H, d)")
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (B, H, Tl):
        raise ValueError("out, dout (B, T/P, H, d) and lse (B, H, T/P) expected")
    gdt = torch.float32 if (flags & ATTN_OUT_F32) else torch.bfloat16
    dq = torch.empty(q.shape, dtype=gdt, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=gdt, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=gdt, device=q.device) if dv is None else dv
    args = (_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
            _dev(out, "out", torch.bfloat16), _dev(dout, "dout", torch.bfloat16), _dev(lse, "lse", torch.float32),
            _dev(dq, "dq", gdt), _dev(dk, "dk", gdt), _dev(dv, "dv", gdt), B, H, T, d, P, rank, int(zigzag),
            int(causal), _dev(kpm, "kpm"), float(rope_base), ATTN_BF16, int(flags))
    var, _keep = _variant(window, alibi_slopes, H)
    if var is None:
        rc = load().attn_ring_bwd(*args, _stream(stream))
    else:
        rc = load().attn_ring_bwd_ex(*args, var, _stream(stream))
    check(rc)
    return dq, dk, dv


def release_scratch() -> None:
    """Free the scratch buffers the library keeps for the current device
    (attn_release_scratch); waits for the device's work first."""
    check(load().attn_release_scratch())


class KernelTimer:
    """Times every attention-kernel launch the library makes on this thread
    (HIP events on the launch's own stream).  ``ms`` holds the per-launch
    durations after the block exits."""

    def __init__(self, max_launches: int = 4096):
        self.max_launches = max_launches
        self.ms: List[float] = []

    def __enter__(self):
        check(load().attn_profile_start(self.max_launches))
        return self

    def __exit__(self, *exc):
        buf = (ctypes.c_float * self.max_launches)()
        n = load().attn_profile_stop(buf, self.max_launches)
        if n < 0:
            check(-n)
        self.ms = [buf[i] for i in range(min(n, self.max_launches))]
        return False
