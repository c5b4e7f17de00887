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
    assert run.ctx.stats()["kernel_variant"] == 4  # binary16 matrix-core cell-major kernel
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows")


@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(64, 8, 1), (32, 8, 2), (8, 8, 1), (48, 16, 1), (16, 8, 3)])
def test_rows_f16_matrix_core_shapes(run, n_head, n_head_kv, n_q):
    """Row counts 1..8 per KV head, two head groups, ragged list lengths (not multiples of the
    16-cell chunk), a random mask with hidden keys, lists overlapping across sequences."""
    rng = gen.rng_for(43)
    n_pool = 2000
    lengths = (300, 1000, 777)
    q = gen.draw_normal(rng, (3, n_head, n_q, 128)).astype(np.float16)
    k = gen.pack_f16(gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    v = gen.pack_f16(gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    rows = gen.rows_lists(rng, n_pool, lengths, 1000, shuffle=True)
    mask = np.stack([gen.random_mask_f16(rng, n_q, 1000, p_hidden=0.25) for _ in range(3)])[:, None]
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=mask, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16,
             scale=1 / np.sqrt(128))
    step(f"rows f16 heads {n_head}/{n_head_kv} n_q={n_q} lists {lengths}")
    O, L = run.rows(w)
    assert run.ctx.stats()["kernel_variant"] == 4
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows f16 mfma")


def test_rows_f16_matrix_core_padding_chunks_and_no_mask(run):
    """Whole 16-entry chunks of padding, padding holes, a list shorter than one chunk."""
    rng = gen.rng_for(44)
    n_pool = 1500
    q = gen.draw_normal(rng, (2, 32, 1, 128)).astype(np.float16)
    k = gen.pack_f16(gen.draw_normal(rng, (n_pool, 8, 128)))
    v = gen.pack_f16(gen.draw_normal(rng, (n_pool, 8, 128)))
    rows = gen.rows_lists(rng, n_pool, (900, 11), 900)
    rows[0, 32:80] = -1
    rows[0, rng.random(900) < 0.2] = -1
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=None, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16,
             scale=1 / np.sqrt(128))
    step("rows f16 padding chunks, 11-entry list, no mask")
    O, L = run.rows(w, mask=None)
    Oref, Lref = oracle_rows(w, mask=None)
    assert_close(O, L, Oref, Lref, what="rows f16 padding")


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


def test_rows_padding_scattered_inside_lists(run):
    """-1 entries in the middle of a list (not only as trailing padding), f16 cell-major pool."""
    rng = np.random.default_rng(17)
    w = gen.make_workload(4, scale_down=16)
    rows = w["kv_rows"].copy()
    hole = rng.random(rows.shape) < 0.3
    rows[hole] = -1
    rows[1, 64:192] = -1  # two whole 64-entry chunks of padding in the middle
    step("rows f16 scattered padding, no mask")
    O, L = run.rows(w, rows=rows, mask=None)
    Oref, Lref = oracle_rows(w, rows=rows, mask=None)
    assert_close(O, L, Oref, Lref, what="rows scattered padding")


@pytest.mark.parametrize("n_head,n_head_kv", [(4, 4), (6, 3), (10, 5)])
def test_rows_head_shapes_without_cell_instantiation(run, n_head, n_head_kv):
    """One row per KV head, or an odd KV head count: the per-head kernel serves these."""
    rng = gen.rng_for(42)
    n_pool = 2500
    q = gen.draw_normal(rng, (3, n_head, 1, 128)).astype(np.float16)
    k = gen.pack_f16(gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    v = gen.pack_f16(gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    rows = gen.rows_lists(rng, n_pool, (900, 400, 1300), 1300)
    mask = np.where(rows[:, None, None, :] >= 0, 0.0, -np.inf).astype(np.float16)
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=mask, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16,
             scale=1 / np.sqrt(128))
    step(f"rows f16 heads {n_head}/{n_head_kv}")
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="rows head shapes")


def test_rows_full_size_config4_all_heads(run):
    """Full pool (65536 cells x 8 KV heads f16) and lists 8192/12288/20480/30720, in the launch
    configuration the benchmark times; the oracle checks every query head of every sequence."""
    import oracle
    w = gen.make_workload(4)
    step("rows full size config 4")
    O, L = run.rows(w)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    gqa = w["n_head"] // w["n_head_kv"]
    mm = np.asarray(w["mask"], dtype=np.float64)[:, 0]
    for g in range(w["n_head_kv"]):
        k = oracle.kv_values(w["k_type"], w["k"][:, g:g + 1])
        v = oracle.kv_values(w["v_type"], w["v"][:, g:g + 1])
        q = np.stack([oracle.q_values(w["q"][b, g * gqa:(g + 1) * gqa]) for b in range(w["q"].shape[0])])
        Oref, Lref = oracle.attention_rows(q, k, v, w["kv_rows"], w["scale"], mm)
        assert_close(O[:, :, g * gqa:(g + 1) * gqa], L[:, :, g * gqa:(g + 1) * gqa], Oref, Lref,
                     what=f"rows full size head group {g}")


@pytest.mark.parametrize("n_head,n_head_kv,kt,vt,variant", [
    (8, 4, gen.TYPE_F16, gen.TYPE_F16, 0),      # per-head vector kernel
    (32, 8, gen.TYPE_F16, gen.TYPE_F16, 4),     # persistent binary16 matrix-core kernel
    (16, 4, gen.TYPE_Q8_0, gen.TYPE_F16, 0),    # per-head vector kernel, q8_0 K
    (32, 8, gen.TYPE_Q8_0, gen.TYPE_Q4_0, 3),   # matrix-core q8_0 / q4_0 kernel
])
def test_rows_entries_outside_the_pool(run, n_head, n_head_kv, kt, vt, variant):
    """List entries >= n_pool are padding on every kernel: nothing is read and the key does not
    count, so the result equals the oracle's for the same list with those entries set to -1."""
    rng = gen.rng_for(61)
    n_pool = 1800
    q = gen.draw_normal(rng, (2, n_head, 1, 128)).astype(np.float16)
    k = gen.pack(kt, gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    v = gen.pack(vt, gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    rows = gen.rows_lists(rng, n_pool, (1000, 700), 1000, shuffle=True)
    bad = (rng.random(rows.shape) < 0.05) & (rows >= 0)
    rows[bad] = n_pool + rng.integers(0, 1 << 20, int(bad.sum()))
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=None, k_type=kt, v_type=vt, n_head=n_head,
             n_head_kv=n_head_kv, scale=1 / np.sqrt(128))
    step(f"rows with entries past the pool: {n_head}/{n_head_kv} types {kt}/{vt}")
    O, L = run.rows(w, mask=None)
    assert run.ctx.stats()["kernel_variant"] == variant
    Oref, Lref = oracle_rows(w, mask=None, rows=np.where(rows < n_pool, rows, -1))
    assert_close(O, L, Oref, Lref, what="rows past the pool")


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0)])
def test_rows_extent_shrinks_between_calls(kt, vt):
    """One context, lists that end earlier (or later) from call to call, down to all padding:
    each call's extent scan bounds the walk by its own lists, so every call matches the oracle."""
    r = Runner()
    try:
        rng = gen.rng_for(77)
        n_pool = 3000
        q = gen.draw_normal(rng, (2, 32, 1, 128)).astype(np.float16)
        k = gen.pack(kt, gen.draw_normal(rng, (n_pool, 8, 128)))
        v = gen.pack(vt, gen.draw_normal(rng, (n_pool, 8, 128)))
        for lengths in ((2500, 2000), (900, 1300), (40, 0), (0, 0), (2400, 17)):
            rows = gen.rows_lists(rng, n_pool, lengths, 2500, shuffle=True)
            w = dict(q=q, k=k, v=v, kv_rows=rows, mask=None, k_type=kt, v_type=vt, scale=1 / np.sqrt(128))
            step(f"rows extent: types {kt}/{vt} lists {lengths} on one context")
            O, L = r.rows(w, mask=None)
            Oref, Lref = oracle_rows(w, mask=None)
            assert_close(O, L, Oref, Lref, what=f"rows extent {lengths}")
            for b, n in enumerate(lengths):
                if n == 0:
                    assert np.all(O[b] == 0) and np.all(L[b] == -np.inf)
    finally:
        r.ctx.close()


def test_rows_more_pairs_than_the_persistent_kernel_plans(run):
    """1100 sequences of one head group (more than the 1024 sequence and head-group pairs the
    persistent binary16 kernel plans): the call falls back to the per-head vector kernel and
    still matches the oracle."""
    rng = gen.rng_for(55)
    n_seq, n_pool = 1100, 300
    lengths = tuple(int(x) for x in rng.integers(0, 24, size=n_seq))
    rows = gen.rows_lists(rng, n_pool, lengths, 24, shuffle=True)
    q = gen.draw_normal(rng, (n_seq, 16, 1, 128)).astype(np.float16)
    k = gen.pack_f16(gen.draw_normal(rng, (n_pool, 8, 128)))
    v = gen.pack_f16(gen.draw_normal(rng, (n_pool, 8, 128)))
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=None, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16, scale=1 / np.sqrt(128))
    step("rows f16: 1100 sequences of 8 KV heads")
    O, L = run.rows(w, mask=None)
    assert run.ctx.stats()["kernel_variant"] == 0
    Oref, Lref = oracle_rows(w, mask=None)
    assert_close(O, L, Oref, Lref, what="rows 1100 sequences")
