"""The matrix-core decode kernel at head dims 64, 256, 512 (dk = dv) and the 576 / 512 pair (q8_0 K
/ q4_0 V, cell-major KV heads) against the fp64 oracle: every head-group size it takes (8 and 4
KV heads at 64; 4, 2 and 1 at 256; 1 at 512 and 576), one to eight rows per KV head and more
in row groups of 16 (several per workgroup at 64, 256 and 512), the window + lifted or device
tail split, masks with an empty row, ragged lengths, the causal rule of a small prefill call,
the soft-cap, and the full 131072-cell shape of the 128K decode at each head dim.  What a
segment computes is the streaming partial of opencoti-llamafile patch 0070-rolling-kv (fattn.cu,
streaming_lse_kernel); the head dims are those its streaming op supports."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, oracle_rows, step

pytestmark = pytest.mark.gpu

MMA = 3  # rkv_kernel_variant: matrix-core cell-major decode


def workload(d, **kw):
    """Workload 2's shape at Q/K head dim d (V head dim 512 with d = 576)."""
    return gen.make_workload(2, d=d, dv=512 if d == 576 else d, **kw)


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)
    r.ctx.set_softcap(0.0)


# (d, n_head, n_head_kv, n_q): the group sizes and 1..8 rows per KV head
SHAPES = [
    (64, 40, 8, 1), (64, 16, 4, 2), (64, 8, 8, 1),
    (256, 40, 8, 1), (256, 8, 2, 2), (256, 3, 1, 2), (256, 7, 1, 1),
    (512, 16, 2, 1), (512, 5, 1, 1), (512, 4, 1, 2), (512, 1, 1, 1),
    (576, 8, 2, 1), (576, 3, 1, 2), (576, 1, 1, 1),
]


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", SHAPES)
def test_groups_and_rows(run, d, n_head, n_head_kv, n_q):
    w = workload(d, scale_down=32, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)  # n_kv 4096
    step(f"mma d={d} heads {n_head}/{n_head_kv} n_q {n_q}: window 2900 + lifted tail in 600-cell tiles")
    O, L = run.decode(w, wc=2900, tile_kv=600, tail="host")
    assert run.ctx.stats()["kernel_variant"] == MMA
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"mma d={d} {n_head}/{n_head_kv} n_q {n_q}")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
@pytest.mark.parametrize("tail", ["device", "host"])
def test_ragged_mask_and_empty_row(run, d, tail):
    w = dict(workload(d, scale_down=32, n_head=16, n_head_kv=4, n_q=2))  # 8 rows per KV head
    n_kv = 3001
    w["k"], w["v"], w["n_kv"] = w["k"][:n_kv], w["v"][:n_kv], n_kv
    mask = gen.random_mask_f16(np.random.default_rng(d), 2, n_kv, p_hidden=0.35)
    mask[1, :] = -np.inf  # the second query sees nothing
    step(f"mma d={d}: n_kv 3001, mask, empty row, {tail} tail")
    O, L = run.decode(w, wc=1999, tile_kv=333, tail=tail, mask=mask)
    assert run.ctx.stats()["kernel_variant"] == MMA
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"mma d={d} mask")
    assert np.all(O[1] == 0) and np.all(L[1] == -np.inf)


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_small_prefill_causal(run, d):
    """Two queries of four heads per KV head (8 rows): the causal rule inside the kernel."""
    w = workload(d, scale_down=32, n_head=16, n_head_kv=4, n_q=2)
    n_q, n_kv = 2, w["n_kv"]
    q_pos0 = n_kv - 700  # the queries sit inside the window, so later keys and the tail are hidden
    step(f"mma d={d}: prefill of 2 queries at {q_pos0}, window 3500 + lifted tail")
    O, L = run.decode(w, wc=3500, tile_kv=300, tail="host", prefill=True, q_pos0=q_pos0)
    assert run.ctx.stats()["kernel_variant"] == MMA
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(n_q, n_kv, q_pos0))
    assert_close(O, L, Oref, Lref, what=f"mma d={d} causal")


# (d, n_head, n_head_kv, n_q): more than 16 rows per KV head, in row groups of 16 (the last one
# ragged), down to a single KV head with 128 query heads; at 64 / 256 / 512 a workgroup takes
# 2 / 4 / 2 row groups over one staged chunk, so the last workgroup can hold empty row groups
# (72 rows at 256: five groups, three of the second workgroup's four empty)
ROW_GROUPS = [(64, 64, 4, 2), (64, 40, 8, 5), (256, 16, 1, 1), (256, 48, 2, 3), (512, 128, 1, 1), (512, 20, 1, 3),
              (576, 128, 1, 1), (576, 16, 1, 2)]


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", ROW_GROUPS)
def test_row_groups(run, d, n_head, n_head_kv, n_q):
    w = workload(d, scale_down=64, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)  # n_kv 2048
    mask = gen.random_mask_f16(np.random.default_rng(d + n_head), n_q, w["n_kv"], p_hidden=0.2)
    step(f"mma d={d} heads {n_head}/{n_head_kv} n_q {n_q} ({n_q * n_head // n_head_kv} rows per KV head)")
    O, L = run.decode(w, wc=1300, tile_kv=400, tail="host", mask=mask)
    assert run.ctx.stats()["kernel_variant"] == MMA
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"mma row groups d={d} {n_head}/{n_head_kv} n_q {n_q}")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_softcap(run, d):
    w = workload(d, scale_down=32, n_head=16, n_head_kv=4)
    run.ctx.set_softcap(20.0)
    try:
        step(f"mma d={d}: soft-cap 20, window 2600 + lifted tail")
        O, L = run.decode(w, wc=2600, tile_kv=512, tail="host")
        assert run.ctx.stats()["kernel_variant"] == MMA
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, softcap=20.0)
    assert_close(O, L, Oref, Lref, what=f"mma d={d} softcap")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_full_size_128k_all_heads(run, d):
    """131072 resident cells, 40/8 heads, in the launch configuration the benchmark times at this
    head dim; every query head against the oracle over all keys."""
    w = workload(d)
    step(f"mma d={d}: full size 131072 cells, 40/8 heads")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    assert run.ctx.stats()["kernel_variant"] == MMA
    gqa = w["n_head"] // w["n_head_kv"]
    for g, (Oref, Lref) in oracle_decode(w, heads=list(range(w["n_head_kv"]))).items():
        assert_close(O[:, g * gqa:(g + 1) * gqa], L[:, g * gqa:(g + 1) * gqa], Oref, Lref, what=f"d={d} head {g}")


# row lists over a q8_0 / q4_0 pool (llama.cpp PR #29510, flash_attn_ext_rows): (d, n_head,
# n_head_kv, n_q)
ROW_LISTS = [(64, 32, 8, 1), (128, 32, 8, 1), (128, 16, 2, 1), (256, 16, 4, 2), (512, 16, 1, 1), (576, 40, 1, 1),
             (64, 96, 4, 1), (256, 32, 1, 1), (512, 40, 1, 1)]  # the last three: several row groups per workgroup


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", ROW_LISTS)
def test_row_lists(run, d, n_head, n_head_kv, n_q):
    """Four shuffled lists with -1 holes, entries past the pool and -1 padding at the end, the
    lists' own mask; an entry past the pool reads nothing, so the oracle takes it as -1."""
    w = gen.make_workload(4, scale_down=16, d=d, dv=512 if d == 576 else d, n_head=n_head, n_head_kv=n_head_kv,
                          n_q=n_q, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)  # pool 4096, lists <= 1920
    rng = np.random.default_rng(d + n_head)
    rows = w["kv_rows"].copy()
    for b in range(rows.shape[0]):
        n = int((rows[b] >= 0).sum())
        rows[b, :n] = rows[b, :n][rng.permutation(n)]
        rows[b, rng.choice(n, size=n // 10, replace=False)] = -1
        rows[b, rng.choice(n, size=3, replace=False)] = w["n_pool"] + 7
    mask = np.where(rng.random((rows.shape[0], 1, n_q, rows.shape[1])) < 0.1, -np.inf, 0.0).astype(np.float16)
    step(f"mma rows d={d} heads {n_head}/{n_head_kv} n_q {n_q}: holes, entries past the pool")
    O, L = run.rows(w, mask=mask, rows=rows)
    assert run.ctx.stats()["kernel_variant"] == MMA
    Oref, Lref = oracle_rows(w, mask=mask, rows=np.where(rows < w["n_pool"], rows, -1))
    assert_close(O, L, Oref, Lref, what=f"mma rows d={d}")


@pytest.mark.parametrize("d", [128, 256])
def test_row_lists_softcap_and_empty_list(run, d):
    """Soft-cap over a q8_0 / q4_0 pool; one sequence's list is all padding (O = 0, LSE = -inf)."""
    w = gen.make_workload(4, scale_down=16, d=d, n_head=32, n_head_kv=8, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    rows = w["kv_rows"].copy()
    rows[2, :] = -1
    run.ctx.set_softcap(25.0)
    try:
        step(f"mma rows d={d}: soft-cap 25, an empty list")
        O, L = run.rows(w, mask=None, rows=rows)
        assert run.ctx.stats()["kernel_variant"] == MMA
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_rows(w, mask=None, rows=rows, softcap=25.0)
    assert_close(O, L, Oref, Lref, what=f"mma rows softcap d={d}")
    assert np.all(O[2] == 0) and np.all(L[2] == -np.inf)
