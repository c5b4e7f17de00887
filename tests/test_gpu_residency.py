"""The position-window residency sizer on the GPU: the device's free memory as the budget,
and a window/tail split chosen by the sizer running through decode against the oracle."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, step

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(scope="module")
def run():
    return Runner()


def test_plan_window_reads_the_device_free_memory(run):
    import torch
    import tiered_kv_cache_split_amd as rkv
    step("plan_window with the device's free memory, capped by a 2 GiB target")
    free, _ = torch.cuda.mem_get_info()
    assert free > 4 * GIB
    # the target caps the budget, so the result does not depend on the exact free figure
    wc = rkv.plan_window(1664, 10**7, -1, 2 * GIB, GIB // 2, 256, ctx=run.ctx)
    assert wc == oracle.plan_window(1664, 10**7, free, 2 * GIB, GIB // 2, 256)
    assert 0 < wc < 10**7 and wc % 256 == 0
    # without a target: the whole of a small cache fits the free memory
    assert rkv.plan_window(1664, 4096, -1, 0, GIB // 2, 256, ctx=run.ctx) == 4096


@pytest.mark.parametrize("n", [1, 2])
def test_sizer_split_through_decode(run, n):
    """A budget of about 60% of the cache: the sizer's window stays on the device, the rest
    is the pinned-host tail, and decode over that split matches the oracle."""
    import tiered_kv_cache_split_amd as rkv
    w = gen.make_workload(n, scale_down=16 if n == 2 else 1)
    n_kv = w["k"].shape[0]
    per_cell = w["k"].shape[1] * w["k"].shape[2] + w["v"].shape[1] * w["v"].shape[2]
    budget = int(0.6 * per_cell * n_kv)
    wc = rkv.plan_window(per_cell, n_kv, budget, 0, 0, 256)
    assert wc == oracle.plan_window(per_cell, n_kv, budget, 0, 0, 256)
    assert rkv.window_mode(rkv.RKV_RESIDENCY_AUTO, wc, n_kv)
    step(f"sizer split workload {n}: wc {wc} of {n_kv} cells")
    O, L = run.decode(w, wc=wc, tile_kv=max(256, (n_kv - wc) // 2))
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"sizer split {n}")
