"""fp64 CPU oracle for split-KV attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``; never by the product path.  It shares no
code with the HIP library.
"""
from .quant import decode, decode_f16, decode_q4_0, decode_q8_0  # noqa: F401
from .attention import (attention, attention_rows, causal_mask, kv_values, merge,  # noqa: F401
                        partial, q_values, scores, split_attention, window_tail_bounds)
from .residency import plan_window, window_mode  # noqa: F401
from .block_cache import ClockCache  # noqa: F401
