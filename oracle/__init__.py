"""Plain float64 CPU oracle of the looped normalized-GPT forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The GPU library never
calls it and shares no code with it.

Source: "Dory1.0-4B: A Looped Normalized-GPT" (paper body page), sections
Architecture, Training with Loops, Long-Context Extension and Last-Loop KV
Caching. Readings of points the pages leave open are listed in `ref.py`'s
module docstring.
"""
from .ref import (  # noqa: F401
    Cache, OracleModel, attention_core, kv_bytes,
    layer_kinds, l2_normalize, ngpt_update, rope, rope_inv_freq, silu,
    swiglu, greedy, sigmoid, softmax_rows, block_of, visible,
)
