"""Head dims other than 128 on the prefill and row-list entry points and with more than eight
rows per KV head, against the fp64 oracle.  Cell-major q8_0 / q4_0 decode, prefill and row lists
run on the matrix-core kernel in row groups of 16; the other type pairs run on the vector kernel
in row groups of eight (opencoti-llamafile patch
0070-rolling-kv: the streaming op's split-and-combine over several head dims; llama.cpp PR
#29510: the row-list form)."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, oracle_rows, step

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (256, 256), (512, 512), (576, 512)]


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)
    r.ctx.set_tail_mode(r.rkv.RKV_TAIL_LIFT)


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("kt,vt", [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0)])
def test_rows(run, dk, dv, kt, vt):
    w = gen.make_workload(4, scale_down=16, d=dk, dv=dv, k_type=kt, v_type=vt)  # pool 4096, lists <= 1920
    step(f"rows head dims {dk}/{dv} types {kt}/{vt}")
    O, L = run.rows(w)
    # q8_0 / q4_0 pools: the matrix-core kernel; binary16 pools of 8 KV heads: the binary16
    # matrix-core kernel
    assert run.ctx.stats()["kernel_variant"] == (3 if kt == gen.TYPE_Q8_0 else 4)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what=f"rows d={dk}/{dv}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (576, 512)])
def test_rows_unsorted_with_holes_and_many_rows(run, dk, dv):
    """Shuffled lists with -1 holes inside, 16 query heads on one KV head (two row groups)."""
    w = gen.make_workload(4, scale_down=16, d=dk, dv=dv, n_head=16, n_head_kv=1)
    rng = np.random.default_rng(dk)
    rows = w["kv_rows"].copy()
    for b in range(rows.shape[0]):
        n = int((rows[b] >= 0).sum())
        perm = rng.permutation(n)
        rows[b, :n] = rows[b, :n][perm]
        rows[b, rng.choice(n, size=n // 10, replace=False)] = -1
    w["kv_rows"] = rows
    w["mask"] = np.where(rows[:, None, None, :] >= 0, 0.0, -np.inf).astype(np.float16)
    step(f"rows head dims {dk}/{dv}: shuffled, holes, 16 rows per KV head")
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what=f"rows holes d={dk}/{dv}")


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("lift", [0, 2])
def test_prefill_causal_window_plus_tail(run, dk, dv, lift):
    w = gen.make_workload(5, scale_down=32, d=dk, dv=dv)  # q8q4, 40/8 heads, n_kv 3328, wc 2048
    n_q = 48
    w["q"] = w["q"][:, -n_q:]
    w["q_pos0"] = w["n_kv"] - n_q
    run.ctx.set_lift_mode(lift)
    step(f"prefill head dims {dk}/{dv}: 48 queries causal, lift {lift}")
    O, L = run.decode(w, tail="host", prefill=True, q_pos0=w["q_pos0"])
    st = run.ctx.stats()
    # 240 rows per KV head over q8_0 / q4_0: the prefill kernel at 64, elsewhere the matrix-core
    # decode kernel in 15 row groups
    assert st["kernel_variant"] == (1 if dk == 64 else 3) and st["n_tail_tiles"] == 2
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(n_q, w["n_kv"], w["q_pos0"]))
    assert_close(O, L, Oref, Lref, what=f"prefill d={dk}/{dv}")


@pytest.mark.parametrize("dk,dv", [(256, 256), (576, 512)])
def test_prefill_mask_only(run, dk, dv):
    w = gen.make_workload(1, d=dk, dv=dv, n_q=9, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_F16)  # 8/2 heads: 36 rows
    mask = gen.random_mask_f16(np.random.default_rng(dk), 9, w["n_kv"], p_hidden=0.3)
    mask[4, :] = -np.inf
    step(f"prefill head dims {dk}/{dv}: mask only, device tail")
    O, L = run.decode(w, wc=1500, tile_kv=1000, tail="device", mask=mask, prefill=True, q_pos0=-1)
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    assert_close(O, L, Oref, Lref, what=f"prefill mask d={dk}/{dv}")
    assert np.all(O[4] == 0) and np.all(L[4] == -np.inf)


@pytest.mark.parametrize("dk,dv", DIMS)
def test_decode_more_than_eight_rows_per_kv_head(run, dk, dv):
    w = gen.make_workload(1, d=dk, dv=dv, n_q=3, n_head=16, n_head_kv=2)  # 24 rows per KV head
    step(f"decode head dims {dk}/{dv}: 24 rows per KV head")
    O, L = run.decode(w, wc=1777, tile_kv=900, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"decode 24 rows d={dk}/{dv}")


def test_prefill_keeps_the_tail_on_the_gpu(run):
    """Prefill computes its tail on the GPU whatever the tail mode, at every head dim."""
    rkv = run.rkv
    w = gen.make_workload(5, scale_down=32, d=64)
    w["q"] = w["q"][:, -8:]
    w["q_pos0"] = w["n_kv"] - 8
    run.ctx.set_tail_mode(rkv.RKV_TAIL_HOST)
    try:
        step("prefill head dim 64 with the host tail mode set")
        O, L = run.decode(w, tail="host", prefill=True, q_pos0=w["q_pos0"])
        assert run.ctx.stats()["tail_host"] == 0
    finally:
        run.ctx.set_tail_mode(rkv.RKV_TAIL_LIFT)
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(8, w["n_kv"], w["q_pos0"]))
    assert_close(O, L, Oref, Lref, what="prefill d=64 tail on the GPU")


def test_rows_q8q4_eight_rows_per_kv_head_at_128(run):
    """Row lists over a q8_0 / q4_0 pool with 8 rows per KV head at head dim 128: the matrix-core
    kernel over groups of 2 KV heads."""
    w = gen.make_workload(4, scale_down=16, n_head=16, n_head_kv=2, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    step("rows q8q4 at 128, 8 rows per KV head")
    O, L = run.rows(w)
    assert run.ctx.stats()["kernel_variant"] == 3
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows q8q4 128 gqa 8")
