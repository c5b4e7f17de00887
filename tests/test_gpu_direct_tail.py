"""The pinned tail read in place (RKV_LIFT_DIRECT): no lift, the segment kernels read the host
copy through its device view.  It is a contrast to the bulk lift (opencoti patch 0102, "bulk-H2D
tail lift": a kernel reading a pinned tail at word granularity is several times slower than a
bulk copy), so only its results are pinned here: decode and prefill against the fp64 oracle,
and the stats report no lift."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    r = Runner()
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_DIRECT)
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)


@pytest.mark.parametrize("layout", ["cell", "head"])
def test_decode_direct_tail(run, layout):
    w = gen.make_workload(3, scale_down=64)  # window 2048, tail 2048, tiles of 512
    step(f"direct tail read: decode {layout}")
    O, L = run.decode(w, tail="host", layout=layout)
    st = run.ctx.stats()
    assert st["lift_mode"] == run.rkv.RKV_LIFT_DIRECT and st["n_tail_tiles"] == 0
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"direct tail {layout}")


def test_decode_direct_tail_masked_ragged(run):
    w = gen.make_workload(3, scale_down=64)
    w["wc"] = 1537  # ragged window end: the tail starts mid tile
    mask = gen.random_mask_f16(np.random.default_rng(21), 1, w["n_kv"], p_hidden=0.3)
    step("direct tail read: ragged window, random mask")
    O, L = run.decode(w, tail="host", mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    assert_close(O, L, Oref, Lref, what="direct tail ragged")


def test_prefill_direct_tail(run):
    w = gen.make_workload(5, scale_down=32)  # n_q 512 -> causal chunk at the end of 3328 cells
    w["q"] = w["q"][:, -96:]
    w["q_pos0"] = w["n_kv"] - 96
    step("direct tail read: prefill causal")
    O, L = run.decode(w, tail="host", prefill=True, q_pos0=w["q_pos0"])
    assert run.ctx.stats()["lift_mode"] == run.rkv.RKV_LIFT_DIRECT
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(96, w["n_kv"], w["q_pos0"]))
    assert_close(O, L, Oref, Lref, what="direct tail prefill")
