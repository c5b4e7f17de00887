"""GPU parity of decode with the tail partial computed on the host cores (RKV_TAIL_HOST):
the window runs on the GPU, the host tail's partial is computed by librkv's host code and
uploaded, and the merge combines both; checked against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_tail_mode(r.rkv.RKV_TAIL_LIFT)


def host_mode(run, n_threads=16):
    run.ctx.set_tail_mode(run.rkv.RKV_TAIL_HOST, n_threads)


@pytest.mark.parametrize("tail", ["host", "pageable"])
def test_config1_host_tail(run, tail):
    host_mode(run)
    w = gen.make_workload(1)
    step(f"decode f16 config1 host tail partial ({tail} memory)")
    O, L = run.decode(w, tail=tail)
    st = run.ctx.stats()
    assert st["tail_host"] == 1 and st["n_tail_tiles"] == 0 and st["lift_bytes"] == 0
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"host tail {tail}")


def test_q8q4_mask_at_global_columns(run):
    host_mode(run, 5)
    w = gen.make_workload(3, scale_down=64)  # n_kv 4096, wc 2048
    w["wc"] = 1333
    rng = np.random.default_rng(2201)
    mask = gen.random_mask_f16(rng, 1, w["n_kv"], p_hidden=0.4)
    step("decode q8q4 host tail partial with mask, wc=1333, pageable tail")
    O, L = run.decode(w, tail="pageable", mask=mask)
    assert run.ctx.stats()["tail_host"] == 1
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="host tail masked")


def test_head_major_tail_and_softcap(run):
    host_mode(run)
    w = gen.make_workload(3, scale_down=64)
    run.ctx.set_softcap(1.5)
    try:
        step("decode q8q4 head-major host tail partial, soft-cap 1.5")
        O, L = run.decode(w, tail="host", layout="head")
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, softcap=1.5)
    assert_close(O, L, Oref, Lref, what="host tail soft-cap")


def test_back_to_back_calls(run):
    """Consecutive calls reuse the context's pinned staging; each result stays correct."""
    host_mode(run)
    ws = [gen.make_workload(3, scale_down=64), gen.make_workload(3, scale_down=32)]
    outs = []
    for i, w in enumerate(ws):
        step(f"decode host tail back-to-back call {i}")
        outs.append(run.decode(w, tail="host"))
    for (O, L), w in zip(outs, ws):
        Oref, Lref = oracle_decode(w)
        assert_close(O, L, Oref, Lref, what="back to back")


def test_device_tail_and_prefill_stay_on_gpu(run):
    host_mode(run)
    w = gen.make_workload(3, scale_down=64)
    step("decode host mode with a device tail")
    O, L = run.decode(w, tail="device")
    assert run.ctx.stats()["tail_host"] == 0
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="device tail in host mode")
    w5 = gen.make_workload(5, scale_down=52)  # 512 queries, n_kv 2048, wc 1260, tiles of 630
    step("prefill in host mode lifts its tail")
    O, L = run.decode(w5, tail="host", prefill=True, q_pos0=w5["q_pos0"])
    st = run.ctx.stats()
    assert st["tail_host"] == 0 and st["n_tail_tiles"] >= 1
    Oref, Lref = oracle_decode(w5, mask=oracle.causal_mask(w5["n_q"], w5["n_kv"], w5["q_pos0"]))
    assert_close(O, L, Oref, Lref, what="prefill in host mode")


def test_full_size_config3_sampled_heads(run):
    """Window 131072 on the GPU, tail 131072 cells (109 MB of q8_0/q4_0) on the host cores."""
    host_mode(run)
    w = gen.make_workload(3)
    step("decode full size config 3, host tail partial")
    O, L = run.decode(w, tail="host")
    st = run.ctx.stats()
    assert st["tail_host"] == 1 and st["host_tail_ms"] > 0
    gqa = w["n_head"] // w["n_head_kv"]
    for g, (Oref, Lref) in oracle_decode(w, heads=[2, 5]).items():
        assert_close(O[:, g * gqa:(g + 1) * gqa], L[:, g * gqa:(g + 1) * gqa], Oref, Lref,
                     what=f"config 3 host tail head {g}")
