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


def test_automatic_mode_reads_small_decode_tails_in_place():
    """RKV_LIFT_AUTO with the default threshold (8 MiB of tail K + V): a small decode tail is read
    in place (no tiles), a larger one lifted with the copy kernel, a decode with more than 8
    rows per KV head and every prefill lifted; the threshold is inclusive and 0 turns it off."""
    import tiered_kv_cache_split_amd as rkv
    from tiered_kv_cache_split_amd import _lib
    r = Runner()  # a context of its own, back to the library's default threshold
    try:
        r.ctx.set_direct_tail_max(8 << 20)
        w1 = gen.make_workload(1)  # 2048-cell binary16 tail, 8/2 heads: 2 MiB
        step("automatic mode: 2 MiB decode tail")
        O, L = r.decode(w1, tail="host")
        st = r.ctx.stats()
        assert st["lift_mode"] == rkv.RKV_LIFT_DIRECT and st["n_tail_tiles"] == 0 and st["lift_bytes"] == 0
        Oref, Lref = oracle_decode(w1)
        assert_close(O, L, Oref, Lref, what="automatic in-place tail")
        tail_bytes = 2048 * 2 * 2 * 256
        r.ctx.set_direct_tail_max(tail_bytes)  # inclusive
        r.decode(w1, tail="host")
        assert r.ctx.stats()["lift_mode"] == rkv.RKV_LIFT_DIRECT
        r.ctx.set_direct_tail_max(tail_bytes - 1)
        step("automatic mode: threshold one byte below the tail")
        O, L = r.decode(w1, tail="host")
        st = r.ctx.stats()
        assert st["lift_mode"] == rkv.RKV_LIFT_KERNEL and st["n_tail_tiles"] == 2
        assert_close(O, L, Oref, Lref, what="automatic lift below threshold")
        r.ctx.set_direct_tail_max(8 << 20)
        w3 = gen.make_workload(3, scale_down=16)  # 8192-cell q8_0 / q4_0 tail, 40/8 heads: 13.6 MB
        step("automatic mode: 13.6 MB decode tail")
        O, L = r.decode(w3, tail="host")
        st = r.ctx.stats()
        assert st["lift_mode"] == rkv.RKV_LIFT_KERNEL and st["n_tail_tiles"] >= 1
        Oref, Lref = oracle_decode(w3)
        assert_close(O, L, Oref, Lref, what="automatic lift of a large tail")
        w6 = gen.make_workload(1, d=64, n_head=32, n_head_kv=2, n_q=1)  # 16 rows per KV head
        step("automatic mode: 16 rows per KV head at head dim 64")
        O, L = r.decode(w6, tail="host")
        assert r.ctx.stats()["lift_mode"] == rkv.RKV_LIFT_KERNEL
        Oref, Lref = oracle_decode(w6)
        assert_close(O, L, Oref, Lref, what="automatic lift with many rows")
        w5 = gen.make_workload(5, scale_down=52)
        step("automatic mode: prefill")
        r.decode(w5, tail="host", prefill=True, q_pos0=w5["q_pos0"])
        assert r.ctx.stats()["lift_mode"] == rkv.RKV_LIFT_BULK
        with pytest.raises(_lib.RkvError):
            r.ctx.set_direct_tail_max(-1)
    finally:
        r.ctx.close()
