"""MI355X (gfx950) forward pass of the looped normalized-GPT: a C-ABI
library of hand-written HIP kernels (libdory.so, built from csrc/) and a thin
Python binding over it. See include/dory.h for the ABI."""
from . import _lib  # noqa: F401
from .model import (KVCache, Model, debug_attention, debug_kv_slots, debug_mask, greedy,  # noqa: F401
                    kv_bytes, schedule, workspace_bytes)
