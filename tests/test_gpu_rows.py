"""GPU parity of rkv_attn_rows (unified pool, kv_rows with -1 padding) against the oracle."""
import numpy as np
import pytest

import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_rows, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    return Runner()


def test_rows_config4_scaled(run):
    w = gen.make_workload(4, scale_down=16)  # pool 4096, lists 512/768/1280/1920 padded to 1920
    step("rows f16 pool=4096 4 seqs padded, mask given")
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows")


def test_rows_padding_ignored_without_mask(run):
    """A negative row contributes nothing whatever the mask says (here: no mask)."""
    w = gen.make_workload(4, scale_down=16)
    step("rows no mask")
    O, L = run.rows(w, mask=None)
    Oref, Lref = oracle_rows(w, mask=None)
    assert_close(O, L, Oref, Lref, what="rows nomask")
    Og, Lg = oracle_rows(w)
    assert_close(O, L, Og, Lg, what="rows nomask == masked")


def test_rows_shuffled_order_and_quant(run):
    rng = np.random.default_rng(4)
    w = gen.make_workload(4, scale_down=16, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    rows = w["kv_rows"].copy()
    for b in range(rows.shape[0]):
        L = int((rows[b] >= 0).sum())
        rows[b, :L] = rng.permutation(rows[b, :L])
    step("rows q8q4 shuffled")
    O, L = run.rows(w, rows=rows)
    Oref, Lref = oracle_rows(w, rows=rows)
    assert_close(O, L, Oref, Lref, what="rows shuffled")


def test_rows_fully_padded_sequence(run):
    w = gen.make_workload(4, scale_down=16)
    rows = w["kv_rows"].copy()
    rows[2, :] = -1
    step("rows one sequence all padding")
    O, L = run.rows(w, rows=rows, mask=None)
    assert np.all(O[2] == 0) and np.all(L[2] == -np.inf)
    Oref, Lref = oracle_rows(w, rows=rows, mask=None)
    assert_close(O, L, Oref, Lref, what="rows all padding")


def test_rows_gqa8_two_queries(run):
    rng = gen.rng_for(41)
    n_pool = 3000
    q = gen.draw_normal(rng, (2, 8, 2, 128)).astype(np.float16)  # gqa 4 x n_q 2 = 8 rows
    k = gen.pack_f16(gen.draw_normal(rng, (n_pool, 2, 128)))
    v = gen.pack_f16(gen.draw_normal(rng, (n_pool, 2, 128)))
    rows = gen.rows_lists(rng, n_pool, (1000, 700), 1000)
    mask = gen.random_mask_f16(rng, 2, 1000, p_hidden=0.2)[None, None].repeat(2, 0)
    mask = np.where(rows[:, None, None, :] >= 0, mask, -np.inf).astype(np.float16)
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=mask, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16,
             scale=1 / np.sqrt(128))
    step("rows gqa4 n_q=2")
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows n_q 2")
