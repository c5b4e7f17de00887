"""Logit soft-cap (scale*qk -> c*tanh(scale*qk/c) before the mask) through every kernel family
against the fp64 oracle: matrix-core decode (q8_0/q4_0 and binary16, window + lifted tail),
the vector decode kernels, row lists, single partials and the prefill kernel."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, oracle_rows, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_softcap(0.0)


@pytest.fixture
def capped(run):
    def set_cap(c):
        run.ctx.set_softcap(c)
    yield set_cap
    run.ctx.set_softcap(0.0)


@pytest.mark.parametrize("num,sd,cap,kernel", [(1, 1, 1.5, 2), (2, 16, 2.0, 3), (2, 16, 0.7, 3)])
def test_softcap_decode_window_and_tail(run, capped, num, sd, cap, kernel):
    w = gen.make_workload(num, scale_down=sd)
    capped(cap)
    step(f"softcap {cap} decode workload {num} (window {w['wc']} + tail)")
    O, L = run.decode(w)
    assert run.ctx.stats()["kernel_variant"] == kernel
    Oref, Lref = oracle_decode(w, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"softcap decode {num}")
    # the cap changes the result: the uncapped oracle is far off
    O0, _ = oracle_decode(w)
    assert np.abs(O0 - Oref).max() > 10 * 2e-3


def test_softcap_decode_binary16_eight_heads_with_mask(run, capped):
    rng = gen.rng_for(71)
    w = gen.make_workload(1, n_head=32, n_head_kv=8)
    mask = gen.random_mask_f16(rng, 1, w["n_kv"], p_hidden=0.3)
    capped(2.5)
    step("softcap 2.5 binary16 decode 32/8 heads, random mask")
    O, L = run.decode(w, mask=mask)
    assert run.ctx.stats()["kernel_variant"] == 4
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64), softcap=2.5)
    assert_close(O, L, Oref, Lref, what="softcap f16 mask")


def test_softcap_outlier_keys_saturate(run, capped):
    """Logits 30x the usual size: most capped scores sit at +-c, where a wrong tanh
    saturation shows."""
    w = gen.make_workload(2, scale_down=16)
    w["scale"] = w["scale"] * 30.0
    capped(3.0)
    step("softcap 3.0 decode q8q4 with large scores")
    O, L = run.decode(w)
    Oref, Lref = oracle_decode(w, softcap=3.0)
    assert_close(O, L, Oref, Lref, what="softcap saturation")


def test_softcap_head_major_vector_kernel(run, capped):
    w = gen.make_workload(2, scale_down=32)
    capped(1.0)
    step("softcap 1.0 decode q8q4 head-major (per-head vector kernel)")
    O, L = run.decode(w, layout="head")
    assert run.ctx.stats()["kernel_variant"] == 0
    Oref, Lref = oracle_decode(w, softcap=1.0)
    assert_close(O, L, Oref, Lref, what="softcap head-major")


def test_softcap_rows(run, capped):
    w = gen.make_workload(4, scale_down=16)
    capped(1.5)
    step("softcap 1.5 rows (binary16 pool, padded lists)")
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w, softcap=1.5)
    assert_close(O, L, Oref, Lref, what="softcap rows")


def test_softcap_prefill_causal(run, capped):
    base = gen.WORKLOADS[5]
    w = gen.make_workload(5, scale_down=max(1, base["n_kv"] // 1664), n_q=96)
    w["wc"], w["tile_kv"] = min(1024, w["n_kv"]), 512
    w["q_pos0"] = w["n_kv"] - 96
    capped(2.0)
    step("softcap 2.0 prefill q8q4 causal chunk, window + tail")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    m = oracle.causal_mask(96, w["n_kv"], w["q_pos0"])
    Oref, Lref = oracle_decode(w, mask=m, softcap=2.0)
    assert_close(O, L, Oref, Lref, what="softcap prefill")


def test_softcap_rejects_bad_values(run):
    import tiered_kv_cache_split_amd as rkv
    for bad in (-1.0, float("inf"), float("nan")):
        with pytest.raises(rkv.RkvError):
            run.ctx.set_softcap(bad)
