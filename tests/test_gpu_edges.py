"""Degenerate and boundary cases of the window + tail split against the fp64 oracle: the whole
cache in the tail (wc = 0), an empty cache (n_kv = 0: every row O = 0, LSE = -inf), one-cell
tiles through the 2-slot ring, and a call in which every key is masked; each with both lift
engines where a tail is lifted."""
import numpy as np
import pytest

import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu

LIFTS = [0, 2]  # DMA engine, copy kernel


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)


@pytest.mark.parametrize("lift", LIFTS)
@pytest.mark.parametrize("num,sd", [(1, 1), (3, 64)])
def test_whole_cache_in_the_tail(run, lift, num, sd):
    w = gen.make_workload(num, scale_down=sd)
    w["wc"] = 0
    run.ctx.set_lift_mode(lift)
    step(f"edge: wc=0 workload {num}/{sd} lift {lift}")
    O, L = run.decode(w, tail="host")
    st = run.ctx.stats()
    assert st["splits_window"] == 0 and st["n_tail_tiles"] == -(-w["n_kv"] // w["tile_kv"])
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="wc=0")


@pytest.mark.parametrize("lift", LIFTS)
def test_one_cell_tiles(run, lift):
    w = gen.make_workload(3, scale_down=1024)  # n_kv 256, wc 128
    w["wc"], w["tile_kv"] = 91, 1  # 165 one-cell tiles through two ring slots
    run.ctx.set_lift_mode(lift)
    step(f"edge: tile_kv=1, 165 tiles, lift {lift}")
    O, L = run.decode(w, tail="host")
    assert run.ctx.stats()["n_tail_tiles"] == 165
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="tile_kv=1")


def test_empty_cache():
    """n_kv = 0: no window cells and no tail; every row gets O = 0 and LSE = -inf."""
    import torch
    import tiered_kv_cache_split_amd as rkv
    ctx = rkv.Context(0)
    try:
        q = dev(np.random.default_rng(3).standard_normal((8, 1, 128)).astype(np.float16))
        kw = torch.empty((0, 2, 256), dtype=torch.uint8, device="cuda")
        o = torch.full((1, 8, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((1, 8), 0.0, dtype=torch.float32, device="cuda")
        step("edge: n_kv = 0")
        ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kw, gen.TYPE_F16), rkv.kv_desc(kw, gen.TYPE_F16), None, None, None,
                        0, 1024, 0.088, o, lse)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(lse == float("-inf"))
    finally:
        ctx.close()


@pytest.mark.parametrize("lift", LIFTS)
def test_every_key_masked(run, lift):
    w = gen.make_workload(3, scale_down=64)
    mask = np.full((1, w["n_kv"]), -np.inf, dtype=np.float16)
    run.ctx.set_lift_mode(lift)
    step(f"edge: every key masked, lift {lift}")
    O, L = run.decode(w, tail="host", mask=mask)
    assert np.all(O == 0) and np.all(L == -np.inf)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="all masked")
