"""CPU fp64 oracle for the KaLM-Reranker-V1 hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the HIP path
computes: chunk pooling, the cross K/V projection, the merged self+cross
attention, the yes/no readout and the decoder-stack glue that chains them,
plus the optional model-shaped layer parts (RMSNorm, RoPE, gated GELU).
It shares no code with the HIP library and never imports it.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import, call or execute anything in this package; the
product path must never route through it.

Parity pins: every function is pinned in ``tests/test_oracle.py`` against a
closed form, an invariant, a library routine (torch's fp64
``scaled_dot_product_attention``, ``scipy.special.expit``/``softmax``,
``numpy.mean``) or brute-force loops on tiny inputs.  Parity unpinned: none of
the functions; the model-level values of the real checkpoints are out of reach
(no weights or printed logits exist for them).
"""
from .kalm_ref import (  # noqa: F401
    round_bf16, round_f32, chunk_pool, cross_kv, merged_attn, merged_attn_partial,
    yesno_score, rank_topn, pair_layout, decoder_stack, stack_scores,
    rms_norm, rope, gelu_tanh, gated_gelu,
)
