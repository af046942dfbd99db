"""Seeded synthetic workloads for blockwise online-softmax attention.

This module only draws inputs: shapes, seeds, value distributions and
key-padding lengths.  It holds none of the attention arithmetic, so both the
fp64 oracle (under ``oracle/``) and the HIP library can be fed from it without
sharing any of the method's code.

Every tensor is drawn per token chunk from its own seed, so the rows of any
chunk (and therefore any ring rank's share) can be regenerated without drawing
the whole sequence:

    seed(cfg, tensor_id, chunk_id) = (1000 + cfg) * 1_000_003 + tensor_id * 1009 + chunk_id

tensor_id: 0 = q, 1 = k, 2 = v, 3 = key-padding lengths.  Values are drawn in
float32 from N(0, sigma^2) and rounded once (round-to-nearest-even) to the
workload dtype; the same rounded values go to the GPU and, widened to float64,
to the oracle.

Workloads 0-4 are the shapes the attention-forward measurements are quoted
on (a small fp32 case, a GPT-2-small-shaped causal case with key padding, an
8K ring-attention share, a 16K bidirectional encoder with key padding, and
one rank's zigzag share of an 8-way ring at 128K context); 5 is one decoding
step over a static cache, and 6 one rank's share of the same 128K sequence
under the head-parallel layout (4 of 32 heads, every token).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Sequence, Tuple

import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_LEN = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    dtype: str                 # "f32" or "bf16"
    B: int
    H: int
    T: int                     # full sequence length
    d: int
    causal: bool
    rope_base: float           # 0 = no rotary embedding
    sigma: float               # std-dev of q, k, v entries
    kpm_len_range: Optional[Tuple[int, int]]  # inclusive range of valid key lengths
    ring_P: int                # number of ranks in the emulated ring (1 = one call)
    ring_rank: int             # which rank's share is computed
    zigzag: bool               # zigzag (2P chunks) vs contiguous (P chunks) placement
    chunk: int                 # token granularity of the seeded draws
    decode: bool = False       # one decoding step over a static cache of T slots per row
                               # (kpm_len_range: filled slots per row; q is one token per row)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def n_chunks(self) -> int:
        return self.T // self.chunk

    def with_heads(self, H: int) -> "Workload":
        """Same workload with fewer heads (heads are the batch axis of the
        method; the first ``H`` heads of each draw are kept)."""
        return replace(self, H=H)


WORKLOADS = {
    0: Workload(0, "attn_fwd_f32_1x2x256_d64_causal", "f32", 1, 2, 256, 64, True, 0.0, 1.0,
                None, 1, 0, False, 256),
    1: Workload(1, "gpt2s_mha_fwd_bf16_4x12x1024_d64_causal_kpm", "bf16", 4, 12, 1024, 64, True, 0.0, 1.0,
                (512, 1024), 1, 0, False, 1024),
    2: Workload(2, "ring_share_bf16_h32_d128_T8192_P4_rank3_causal_rope", "bf16", 1, 32, 8192, 128, True,
                10000.0, 1.0, None, 4, 3, False, 2048),
    3: Workload(3, "encoder_fwd_bf16_2x16x16384_d128_kpm", "bf16", 2, 16, 16384, 128, False, 0.0, 0.5,
                (12288, 16384), 1, 0, False, 4096),
    4: Workload(4, "zigzag_ring_share_bf16_h32_d128_T131072_P8_rank0_causal_rope", "bf16", 1, 32, 131072,
                128, True, 10000.0, 1.0, None, 8, 0, True, 8192),
    5: Workload(5, "decode_step_bf16_b8_h32_d128_cache32768_rope", "bf16", 8, 32, 32768, 128, True, 10000.0,
                1.0, (16384, 32000), 1, 0, False, 4096, decode=True),
    # one rank's share under the head-parallel (Ulysses) layout of the same
    # 128K sequence: after the all-to-all a rank holds H/P = 32/8 heads of
    # every token, so its attention is one call over the whole sequence
    6: Workload(6, "ulysses_share_bf16_h4_d128_T131072_causal_rope", "bf16", 1, 4, 131072, 128, True, 10000.0,
                1.0, None, 1, 0, False, 8192),
}


def seed_for(w: Workload, tensor_id: int, chunk_id: int) -> int:
    return (1000 + w.index) * 1_000_003 + tensor_id * 1009 + chunk_id


def draw_chunk(w: Workload, tensor_id: int, chunk_id: int, heads: Optional[int] = None) -> torch.Tensor:
    """One chunk of q (0), k (1) or v (2): shape (B, chunk, H, d) in the
    workload dtype, on the CPU.  ``heads`` keeps only the first heads."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(w, tensor_id, chunk_id))
    x = torch.randn((w.B, w.chunk, w.H, w.d), generator=g, dtype=torch.float32)
    if w.sigma != 1.0:
        x.mul_(w.sigma)
    if heads is not None and heads < w.H:
        x = x[:, :, :heads, :].contiguous()
    return x.to(w.torch_dtype)


def draw_tokens(w: Workload, tensor_id: int, chunk_ids: Sequence[int], heads: Optional[int] = None) -> torch.Tensor:
    """Concatenation (along tokens) of the given chunks."""
    return torch.cat([draw_chunk(w, tensor_id, c, heads) for c in chunk_ids], dim=1).contiguous()


def kpm_lengths(w: Workload) -> Optional[torch.Tensor]:
    """Valid key length L_b per batch item, uniform over the inclusive range."""
    if w.kpm_len_range is None:
        return None
    lo, hi = w.kpm_len_range
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(w, TENSOR_LEN, 0))
    return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)


def key_padding_mask(w: Workload, T: Optional[int] = None) -> Optional[torch.Tensor]:
    """uint8 (B, T): 1 marks a padded (ignored) key, i.e. keys [L_b, T)."""
    lens = kpm_lengths(w)
    if lens is None:
        return None
    T = w.T if T is None else T
    idx = torch.arange(T).unsqueeze(0)
    return (idx >= lens.unsqueeze(1)).to(torch.uint8).contiguous()


def random_normal(shape, seed: int, dtype: torch.dtype = torch.float32, sigma: float = 1.0) -> torch.Tensor:
    """Generic seeded N(0, sigma^2) draw, rounded once to ``dtype`` (used by
    the edge-case tests for shapes outside the five workloads)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def alibi_slopes(H: int) -> torch.Tensor:
    """Per-head ALiBi slopes used as test and bench inputs: the geometric
    sequence 2^(-8 h / H), h = 1 .. H, of the ALiBi paper (the digest entry
    only says each head has a fixed slope), as float32."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def random_mask(shape, seed: int, p: float) -> torch.Tensor:
    """Seeded Bernoulli(p) uint8 mask (1 = excluded)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.rand(tuple(shape), generator=g) < p).to(torch.uint8).contiguous()
