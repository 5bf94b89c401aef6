"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path never does: it shares
no code, tables or helpers with it.

Pinned by the tests under ``tests/test_oracle_*.py`` against the worked examples,
closed forms, invariants, library routines and finite differences listed there.
Parity status: every function is pinned (no "parity unpinned" entry).
"""
from .attention import attention_fwd, attention_bwd, visible_mask
from .online import online_softmax, three_pass_softmax_average, merge, tiled_forward
from .splitkv import (attention_fwd_rect, merge_partials, split_ranges, splitkv_partials,
                      visible_rect)

__all__ = [
    "attention_fwd", "attention_bwd", "visible_mask",
    "online_softmax", "three_pass_softmax_average", "merge", "tiled_forward",
    "attention_fwd_rect", "merge_partials", "split_ranges", "splitkv_partials", "visible_rect",
]
