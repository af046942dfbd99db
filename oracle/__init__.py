"""fp64 CPU oracle for blockwise online-softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (no kernels, headers, helpers or tables) and the
library never imports it.

Every function states the passage of the source pages it follows:

* "Transformers and Attention" (ai.engineer topic digest), numbered references
  #2 (PyTorch MultiheadAttention masks), #4 (RoFormer), #15/#22 (Attention Is
  All You Need), #18 (Set Transformer), #24 (PyTorch scaled_dot_product_attention);
* "CP: Split Long Contexts Across GPUs" (llm-systems-engineering.pages.dev):
  sections "Why attention needs information from other GPUs", "Circulate K/V
  blocks with Ring", "Balance the workload in causal attention";
* the sequence/context-parallelism post on brunomaga.github.io: section "Ring
  Attention" (fraction form), "Improving numerical stability" (safe softmax,
  accumulator rescale, LogSumExp), "Distributed algorithm" and "Implementation"
  (forward and backward pass of the ring);
* "Transformers and Attention" #53 (causal key/value caching), #55
  (Longformer sliding windows), #57 (static caches and windowed retention),
  #58 (ALiBi) for the variants: window, linear distance bias, decoding.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
facts the pages or mathematics fix (printed worked example, closed forms,
invariants, library special cases, brute force).  The RoPE pairing and
frequency schedule (adjacent pairs, theta_t = base^(-2t/d), a reading of
"Transformers and Attention" #4) are pinned against the interleaved rotary
routine of the GPT-J model in the installed ``transformers`` package.
"""
from .reference import (  # noqa: F401
    round_to_dtype,
    rope_rotate,
    rope_frequencies,
    sdpa,
    sdpa_backward,
    key_block_gradients,
    attention,
    attention_backward,
    alibi_bias,
    kv_append,
    decode,
    merge,
    ring_order,
    zigzag_chunks,
    local_query_positions,
    allowed_pairs,
    zigzag_pairs_closed_form,
)
