"""Oracle: residency sizing of the rolling-KV position window and the window-mode rule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never calls it.

Source: opencoti-llamafile patch 0070-rolling-kv, KV-cache hunk -- the position-axis
residency sizer (how many leading cells fit the device budget; the rest is the
pinned-host tail) and the residency-mode eligibility rule that follows it.  The steps
are taken in the page's order:

1. budget = free device bytes, capped at the target when one is given, minus a fixed
   reserve (never below zero);
2. the whole cache fits the budget -> every cell resident (no tail);
3. otherwise the largest cell count that fits, rounded down to the alignment, never
   below one alignment unit, and never so large that less than one unit of tail is
   left (that cap is itself rounded down to the alignment).

Reading taken where the page is silent: the result never exceeds the cache size (a
cache shorter than one alignment unit that does not fit is kept resident).
"""


def plan_window(per_cell: int, kv_size: int, free_bytes: int, target_bytes: int,
                reserve_bytes: int, align: int) -> int:
    """Resident cell count wc of a cache of kv_size cells, per_cell bytes per cell."""
    if kv_size == 0:
        return 0
    budget = free_bytes
    if target_bytes > 0:
        budget = min(budget, target_bytes)
    budget = budget - reserve_bytes if budget > reserve_bytes else 0
    if per_cell * kv_size <= budget:
        return kv_size
    cells = (budget // per_cell) // align * align
    if cells < align:
        cells = align
    if kv_size > align and cells > kv_size - align:
        cells = (kv_size - align) // align * align
        if cells < align:
            cells = align
    return min(cells, kv_size)


def window_mode(mode: int, wc: int, kv_size: int, append_only: bool, v_transposed: bool) -> bool:
    """Whether the cache runs as window + tail.  mode 0 = auto (window when eligible),
    1 = never window, 2 = window when eligible (otherwise resident).  Eligible: the sizer
    found a real overflow (0 < wc < kv_size) on a cache whose cell index is the key
    position (append-only) and whose V is not transposed."""
    eligible = 0 < wc < kv_size and append_only and not v_transposed
    return bool(eligible and mode != 1)
