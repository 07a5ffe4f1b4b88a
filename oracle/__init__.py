"""fp64 CPU oracle for causal self-attention — TEST INFRASTRUCTURE ONLY.

Only `tests/`, the graft entry's smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never imports it and has no CPU fallback.

Every function is pinned by the CPU tests in tests/test_oracle.py (finite
differences, closed forms, invariants and an independent library routine);
no function is "parity unpinned".
"""
from .attention import (  # noqa: F401
    softmax_scale, forward_head, backward_head, forward, backward,
    decode_head, decode, causal_probabilities, kv_head, kv_grads, prefill_head, prefill,
)
from .prologue import (  # noqa: F401
    rope_tables, qk_norm_rope_forward, qk_norm_rope_backward, value_gate_forward,
    value_gate_backward,
)
