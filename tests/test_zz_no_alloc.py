"""attn_decode_noalloc (GPU): the decode entry point that allocates nothing.

Its chunk partials live in the library's per-device static workspace instead
of stream-ordered scratch; the kernels are attn_decode's, so its out and lse
must equal attn_decode's bit for bit.  Two calls in a row on the same device,
the second smaller than the first, so the second runs over a workspace that
still holds the first call's partials.
"""
from __future__ import annotations

import pytest
import torch

import blockwise_online_softmax_attn_amd as bosa
import workloads
from gpu_helpers import DEV, note

pytestmark = pytest.mark.gpu


def _case(B, H, Tcap, d, dtype, seed, rope, window_left, alibi):
    kc = workloads.random_normal((B, Tcap, H, d), seed, dtype).to(DEV)
    vc = workloads.random_normal((B, Tcap, H, d), seed + 1, dtype).to(DEV)
    q = workloads.random_normal((B, H, d), seed + 2, dtype).to(DEV)
    g = torch.Generator().manual_seed(seed + 3)
    lens = torch.randint(0, Tcap + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = Tcap                      # one full row
    if B > 2:
        lens[1] = 0                     # and one empty row
    slopes = workloads.alibi_slopes(H).to(DEV) if alibi else None
    return q, kc, vc, lens.to(DEV), slopes


@pytest.mark.parametrize("first,second", [
    ((8, 32, 8192, 128, torch.bfloat16, 10000.0, -1, False), (3, 4, 1500, 64, torch.float32, 500.0, 300, True)),
    ((16, 64, 4096, 128, torch.bfloat16, 10000.0, 1000, True), (2, 2, 700, 128, torch.bfloat16, 0.0, -1, False)),
])
def test_decode_noalloc_matches_decode_twice(first, second):
    for i, (B, H, Tcap, d, dtype, rope, wl, alibi) in enumerate((first, second)):
        note(f"decode_noalloc call {i}: B={B} H={H} Tcap={Tcap} d={d} {dtype} rope={rope} window_left={wl} "
             f"alibi={alibi}")
        q, kc, vc, lens, slopes = _case(B, H, Tcap, d, dtype, 9100 + 10 * i, rope, wl, alibi)
        out_a = torch.empty((B, H, d), dtype=dtype, device=DEV)
        lse_a = torch.empty((B, H), dtype=torch.float32, device=DEV)
        out_b = torch.empty_like(out_a)
        lse_b = torch.empty_like(lse_a)
        bosa.attn_decode(q, kc, vc, lens, out_a, lse_a, rope_base=rope, window_left=wl, alibi_slopes=slopes)
        bosa.attn_decode(q, kc, vc, lens, out_b, lse_b, rope_base=rope, window_left=wl, alibi_slopes=slopes,
                         noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(out_a.cpu(), out_b.cpu()), f"call {i}: out differs"
        assert torch.equal(lse_a.cpu(), lse_b.cpu()), f"call {i}: lse differs"
        if B > 2:
            assert torch.isneginf(lse_b[1]).all() and not out_b[1].float().abs().any()


def test_decode_noalloc_rejects_a_call_beyond_its_workspace():
    """Partials of 40000 rows at d = 128 need about 20 MB: rejected before
    anything is enqueued, with the limit in the message."""
    B, H, Tcap, d = 1, 40000, 1, 128
    kc = torch.zeros((B, Tcap, H, d), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    with pytest.raises(bosa.AttnError) as ei:
        bosa.attn_decode(q, kc, kc, lens, noalloc=True)
    assert ei.value.code == bosa._lib.ATTN_ERR_UNSUPPORTED
    assert "static workspace" in str(ei.value)
