"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/attn.h declares, rejects bad arguments before any HIP
call, and plans ring shares that cover exactly the pairs the oracle's own
bookkeeping says a rank must see."""
import ctypes
import os
import re

import numpy as np
import pytest

import blockwise_online_softmax_attn_amd as bosa
from blockwise_online_softmax_attn_amd import _lib
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_library_exports_every_declared_symbol():
    lib = bosa.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.attn_version() >= 100


def _fwd(**kw):
    lib = bosa.load()
    a = dict(q=1 << 20, k=1 << 20, v=1 << 20, out=1 << 20, lse=1 << 20, B=1, H=1, Tq=4, Tkv=4, d=64, q_off=0,
             kv_off=0, causal=0, kpm=None, amask=None, rope=0.0, dtype=_lib.ATTN_BF16, flags=0, stream=None)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Tq"], a["Tkv"], a["d"],
                        a["q_off"], a["kv_off"], a["causal"], a["kpm"], a["amask"], a["rope"], a["dtype"],
                        a["flags"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(d=0), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(Tkv=-3), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(out=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(k=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q=(1 << 20) + 2), _lib.ATTN_ERR_INVALID_ARG),
    (dict(flags=64), _lib.ATTN_ERR_INVALID_ARG),
    (dict(flags=_lib.ATTN_ACCUMULATE), _lib.ATTN_ERR_INVALID_ARG),
    (dict(flags=_lib.ATTN_ACCUMULATE | _lib.ATTN_OUT_F32, lse=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(rope=-1.0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(rope=float("nan")), _lib.ATTN_ERR_INVALID_ARG),
    (dict(rope=float("inf")), _lib.ATTN_ERR_INVALID_ARG),
])
def test_attn_fwd_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code
    assert bosa.load().attn_last_error()


def test_attn_fwd_empty_problem_is_a_no_op():
    assert _fwd(q=None, out=None, Tq=0) == 0
    assert _fwd(B=0) == 0 and _fwd(H=0) == 0


def test_other_entry_points_reject_bad_arguments():
    lib = bosa.load()
    assert lib.attn_merge(None, None, None, None, 1, 1, 1, 64, _lib.ATTN_F32, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_merge(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1, 1, 1, 66, _lib.ATTN_F32, None) == _lib.ATTN_ERR_UNSUPPORTED
    assert lib.attn_merge(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1, 1, 1, 64, 5, None) == _lib.ATTN_ERR_UNSUPPORTED
    assert lib.rope_apply(1 << 20, 1 << 20, 0.0, 1, 4, 1, 64, _lib.ATTN_BF16, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.rope_apply(1 << 20, 1 << 20, 1e4, 1, 4, 1, 63, _lib.ATTN_BF16, None) == _lib.ATTN_ERR_UNSUPPORTED
    assert lib.rope_apply(None, None, 1e4, 1, 4, 1, 64, _lib.ATTN_BF16, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_cast(None, None, 10, _lib.ATTN_BF16, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_cast(1 << 20, 1 << 20, -1, _lib.ATTN_BF16, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_cast(1 << 20, 1 << 20, 0, _lib.ATTN_BF16, None) == 0
    assert lib.attn_ring_fwd(None, None, None, None, None, None, 1, 1, 100, 64, 3, 0, 0, 1, None, 0.0,
                             _lib.ATTN_BF16, 0, None) == _lib.ATTN_ERR_INVALID_ARG   # 100 % 3 != 0
    assert lib.attn_ring_fwd(None, None, None, None, None, None, 1, 1, 96, 64, 3, 0, 0, 1, None, 0.0,
                             _lib.ATTN_BF16, 0, None) == _lib.ATTN_ERR_INVALID_ARG   # NULL pointers
    assert lib.attn_ring_plan(8, 2, 2, 0, 1, None, 0) < 0                               # rank out of range


def test_decode_noalloc_checks_its_workspace_before_any_hip_call():
    """attn_decode_noalloc validates like attn_decode and rejects partials
    larger than its static workspace on the host (no GPU is touched here)."""
    lib = bosa.load()
    p = 1 << 20
    # 40000 rows of partials at d = 128: about 20 MB, over the 16 MiB workspace
    assert lib.attn_decode_noalloc(p, p, p, p, p, p, 1, 40000, 1, 128, 0.0, _lib.ATTN_BF16, 0, None,
                                   None) == _lib.ATTN_ERR_UNSUPPORTED
    assert b"static workspace" in lib.attn_last_error()
    assert lib.attn_decode_noalloc(p, p, p, p, p, p, 1, 4, 16, 96, 0.0, _lib.ATTN_BF16, 0, None,
                                   None) == _lib.ATTN_ERR_UNSUPPORTED
    assert lib.attn_decode_noalloc(None, p, p, p, p, p, 1, 4, 16, 128, 0.0, _lib.ATTN_BF16, 0, None,
                                   None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_decode_noalloc(p, p, p, p, p, p, 0, 4, 16, 128, 0.0, _lib.ATTN_BF16, 0, None, None) == 0


def _pairs_of_plan(plan, T, P, rank, zigzag, causal):
    """(query position, key position) pairs the plan evaluates."""
    qpos = oracle.local_query_positions(T, P, rank, zigzag)
    seen = []
    for c in plan:
        for i in range(c.q_rows):
            qp = qpos[c.q_row0 + i]
            assert qp == c.q_pos0 + i
            for j in range(c.kv_rows):
                kp = c.kv_pos0 + j
                if not causal or kp <= qp:
                    seen.append((qp, kp))
    return seen


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("zigzag", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_ring_plan_covers_every_allowed_pair_once(P, zigzag, causal):
    T = 2 * P * 3
    for rank in range(P):
        plan = bosa.attn_ring_plan(T, P, rank, zigzag, causal)
        seen = _pairs_of_plan(plan, T, P, rank, zigzag, causal)
        assert len(seen) == len(set(seen))
        qpos = oracle.local_query_positions(T, P, rank, zigzag)
        want = oracle.allowed_pairs(qpos, range(T), causal)
        assert len(seen) == want
        # steps follow the ring order, one block per step
        order = oracle.ring_order(P, rank)
        assert [c.block for c in plan] == sorted([c.block for c in plan], key=lambda b: order.index(b))
        for c in plan:
            assert c.block == order[c.step]
        # the first sub-call touching a query chunk writes, the rest merge
        first = {}
        for c in plan:
            assert c.accumulate == (1 if c.q_row0 in first else 0)
            first.setdefault(c.q_row0, c)


def test_ring_plan_for_the_two_ring_workloads():
    # 8K share, 4 ranks, rank 3, contiguous: blocks 3, 2, 1, 0
    plan = bosa.attn_ring_plan(8192, 4, 3, False, True)
    assert [c.block for c in plan] == [3, 2, 1, 0]
    assert [c.kv_pos0 for c in plan] == [6144, 4096, 2048, 0]
    assert all(c.q_pos0 == 6144 and c.q_rows == 2048 for c in plan)
    # 128K zigzag share, 8 ranks, rank 0: 17 live sub-calls, 15 merges into the late chunk
    plan = bosa.attn_ring_plan(131072, 8, 0, True, True)
    assert len(plan) == 17
    assert [c.block for c in plan][:3] == [0, 0, 0] and plan[3].block == 7
    late = [c for c in plan if c.q_row0 == 8192]
    assert len(late) == 16 and sum(c.accumulate for c in late) == 15
    total = 0
    for c in plan:
        qp0, kp0, n = c.q_pos0, c.kv_pos0, c.q_rows
        if kp0 + n - 1 <= qp0:
            total += n * n
        else:  # diagonal block
            assert kp0 == qp0
            total += n * (n + 1) // 2
    assert total == oracle.zigzag_pairs_closed_form(8, 8192) == 1_073_750_016


def test_variant_and_decode_entry_points_reject_bad_arguments():
    lib = bosa.load()
    P = 1 << 20
    bad_window = _lib.Variant(-2, -1, None)
    assert lib.attn_fwd_ex(P, P, P, P, P, 1, 1, 4, 4, 64, 0, 0, 0, None, None, 0.0, _lib.ATTN_BF16, 0,
                           ctypes.byref(bad_window), None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_fwd_ex(P, P, P, P, P, 1, 1, 4, 4, 96, 0, 0, 0, None, None, 0.0, _lib.ATTN_BF16, 0,
                           None, None) == _lib.ATTN_ERR_UNSUPPORTED
    # decode: head dim, dtype, flags, window, NULL pointers, alignment
    dec = lambda **kw: lib.attn_decode(kw.get("q", P), P, P, kw.get("len", P), kw.get("out", P), None,  # noqa: E731
                                       1, 2, 16, kw.get("d", 128), 0.0, kw.get("dtype", _lib.ATTN_BF16),
                                       kw.get("flags", 0), kw.get("var"), None)
    assert dec(d=80) == _lib.ATTN_ERR_UNSUPPORTED
    assert dec(dtype=3) == _lib.ATTN_ERR_UNSUPPORTED
    assert dec(flags=_lib.ATTN_ACCUMULATE) == _lib.ATTN_ERR_INVALID_ARG
    assert dec(var=ctypes.byref(bad_window)) == _lib.ATTN_ERR_INVALID_ARG
    assert dec(q=None) == _lib.ATTN_ERR_INVALID_ARG
    assert dec(len=None) == _lib.ATTN_ERR_INVALID_ARG
    assert dec(q=P + 8) == _lib.ATTN_ERR_INVALID_ARG
    # append: sizes, dtype, alignment, NULL pointers; empty problems do nothing
    app = lambda **kw: lib.attn_kv_append(kw.get("k", P), P, P, P, kw.get("len", P), kw.get("B", 1), 2, 16,  # noqa: E731
                                          kw.get("d", 64), kw.get("rope", 0.0), kw.get("dtype", _lib.ATTN_F32), None)
    assert app(B=-1) == _lib.ATTN_ERR_INVALID_ARG
    assert app(d=32) == _lib.ATTN_ERR_UNSUPPORTED
    assert app(dtype=9) == _lib.ATTN_ERR_UNSUPPORTED
    assert app(rope=-2.0) == _lib.ATTN_ERR_INVALID_ARG
    assert app(k=None) == _lib.ATTN_ERR_INVALID_ARG
    assert app(k=P + 4) == _lib.ATTN_ERR_INVALID_ARG
    assert app(B=0, k=None, len=None) == 0


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """With libattn.so absent, the loader and the entry points raise: there is
    no CPU path to fall back to."""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="no CPU fallback"):
        _lib.load()
    with pytest.raises(ImportError):
        bosa.attn_ring_plan(8192, 4, 3, False, True)
