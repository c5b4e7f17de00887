"""The binary16 matrix-core decode kernel at head dims 64, 256 and 512 (dk = dv; cell groups of
8, 4 and 2 KV heads, so one, two and four waves per KV head, each with its share of the P.V
tiles) and at the 576 / 512 pair (one KV head per workgroup, eight waves) against the fp64
oracle: several head groups, one to eight rows per KV head, the window
+ lifted or device tail split, masks with an empty row, ragged lengths, the causal rule of a
small prefill call, the soft-cap, the full 131072-cell shape of the 128K decode, and row lists
(holes, entries past the pool, an empty list) over several sequences, so that the persistent
workgroups cross (sequence, head group) boundaries.  What a segment computes is the streaming
partial of opencoti-llamafile patch 0070-rolling-kv (fattn.cu, streaming_lse_kernel), and for
row lists llama.cpp PR #29510's flash_attn_ext_rows; the head dims are those the streaming op
supports."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, oracle_rows, step

pytestmark = pytest.mark.gpu

MMA16 = 4  # rkv_kernel_variant: binary16 matrix-core cell-major decode
F16 = gen.TYPE_F16


def workload(num, d, **kw):
    """Workload `num` with binary16 K and V at Q / K head dim d (V head dim 512 with 576)."""
    return gen.make_workload(num, d=d, dv=512 if d == 576 else d, k_type=F16, v_type=F16, **kw)


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)
    r.ctx.set_softcap(0.0)


# (d, n_head, n_head_kv, n_q): one and several head groups, 1 .. 8 rows per KV head
SHAPES = [
    (64, 40, 8, 1), (64, 64, 16, 2), (64, 8, 8, 1),
    (256, 40, 8, 1), (256, 16, 4, 2), (256, 12, 4, 1),
    (512, 16, 2, 1), (512, 6, 2, 1), (512, 8, 4, 2),
    (576, 16, 2, 1), (576, 3, 1, 2), (576, 8, 1, 1),
]


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", SHAPES)
def test_groups_and_rows(run, d, n_head, n_head_kv, n_q):
    w = workload(2, d, scale_down=32, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)  # n_kv 4096
    step(f"f16 mma d={d} heads {n_head}/{n_head_kv} n_q {n_q}: window 2900 + lifted tail in 600-cell tiles")
    O, L = run.decode(w, wc=2900, tile_kv=600, tail="host")
    assert run.ctx.stats()["kernel_variant"] == MMA16
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"f16 mma d={d} {n_head}/{n_head_kv} n_q {n_q}")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
@pytest.mark.parametrize("tail", ["device", "host"])
def test_ragged_mask_and_empty_row(run, d, tail):
    w = dict(workload(2, d, scale_down=32, n_head=32, n_head_kv=8, n_q=2))  # 8 rows per KV head
    n_kv = 3001
    w["k"], w["v"], w["n_kv"] = w["k"][:n_kv], w["v"][:n_kv], n_kv
    mask = gen.random_mask_f16(np.random.default_rng(d), 2, n_kv, p_hidden=0.35)
    mask[1, :] = -np.inf  # the second query sees nothing
    step(f"f16 mma d={d}: n_kv 3001, mask, empty row, {tail} tail")
    O, L = run.decode(w, wc=1999, tile_kv=333, tail=tail, mask=mask)
    assert run.ctx.stats()["kernel_variant"] == MMA16
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"f16 mma d={d} mask")
    assert np.all(O[1] == 0) and np.all(L[1] == -np.inf)


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_small_prefill_causal(run, d):
    """Two queries of four heads per KV head (8 rows): the causal rule inside the kernel."""
    w = workload(2, d, scale_down=32, n_head=32, n_head_kv=8, n_q=2)
    n_q, n_kv = 2, w["n_kv"]
    q_pos0 = n_kv - 700  # the queries sit inside the window, so later keys and the tail are hidden
    step(f"f16 mma d={d}: prefill of 2 queries at {q_pos0}, window 3500 + lifted tail")
    O, L = run.decode(w, wc=3500, tile_kv=300, tail="host", prefill=True, q_pos0=q_pos0)
    assert run.ctx.stats()["kernel_variant"] == MMA16
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(n_q, n_kv, q_pos0))
    assert_close(O, L, Oref, Lref, what=f"f16 mma d={d} causal")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_softcap(run, d):
    w = workload(2, d, scale_down=32, n_head=16, n_head_kv=8)
    run.ctx.set_softcap(20.0)
    try:
        step(f"f16 mma d={d}: soft-cap 20, window 2600 + lifted tail")
        O, L = run.decode(w, wc=2600, tile_kv=512, tail="host")
        assert run.ctx.stats()["kernel_variant"] == MMA16
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, softcap=20.0)
    assert_close(O, L, Oref, Lref, what=f"f16 mma d={d} softcap")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_full_size_128k(run, d):
    """131072 resident cells, 40/8 heads, in the launch configuration of the 128K decode at this
    head dim; the query heads of KV heads 0, 3 and 7 against the oracle over all keys."""
    w = workload(2, d)
    step(f"f16 mma d={d}: full size 131072 cells, 40/8 heads")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    assert run.ctx.stats()["kernel_variant"] == MMA16
    gqa = w["n_head"] // w["n_head_kv"]
    for g, (Oref, Lref) in oracle_decode(w, heads=[0, 3, 7]).items():
        assert_close(O[:, g * gqa:(g + 1) * gqa], L[:, g * gqa:(g + 1) * gqa], Oref, Lref, what=f"d={d} head {g}")


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", [(64, 32, 8, 1), (256, 32, 8, 1), (256, 16, 4, 2), (512, 16, 8, 1),
                                                    (512, 8, 2, 1), (576, 16, 2, 1), (576, 8, 1, 1)])
def test_row_lists(run, d, n_head, n_head_kv, n_q):
    """Four shuffled lists with -1 holes, entries past the pool and -1 padding at the end, the
    lists' own mask; an entry past the pool reads nothing, so the oracle takes it as -1."""
    w = workload(4, d, scale_down=16, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)  # pool 4096, lists <= 1920
    rng = np.random.default_rng(d + n_head)
    rows = w["kv_rows"].copy()
    for b in range(rows.shape[0]):
        n = int((rows[b] >= 0).sum())
        rows[b, :n] = rows[b, :n][rng.permutation(n)]
        rows[b, rng.choice(n, size=n // 10, replace=False)] = -1
        rows[b, rng.choice(n, size=3, replace=False)] = w["n_pool"] + 7
    mask = np.where(rng.random((rows.shape[0], 1, n_q, rows.shape[1])) < 0.1, -np.inf, 0.0).astype(np.float16)
    step(f"f16 mma rows d={d} heads {n_head}/{n_head_kv} n_q {n_q}: holes, entries past the pool")
    O, L = run.rows(w, mask=mask, rows=rows)
    assert run.ctx.stats()["kernel_variant"] == MMA16
    Oref, Lref = oracle_rows(w, mask=mask, rows=np.where(rows < w["n_pool"], rows, -1))
    assert_close(O, L, Oref, Lref, what=f"f16 mma rows d={d}")


@pytest.mark.parametrize("d", [64, 512, 576])
def test_row_lists_softcap_and_empty_list(run, d):
    """Soft-cap over a binary16 pool; one sequence's list is all padding (O = 0, LSE = -inf)."""
    w = workload(4, d, scale_down=16, n_head=32, n_head_kv=8)
    rows = w["kv_rows"].copy()
    rows[2, :] = -1
    run.ctx.set_softcap(25.0)
    try:
        step(f"f16 mma rows d={d}: soft-cap 25, an empty list")
        O, L = run.rows(w, mask=None, rows=rows)
        assert run.ctx.stats()["kernel_variant"] == MMA16
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_rows(w, mask=None, rows=rows, softcap=25.0)
    assert_close(O, L, Oref, Lref, what=f"f16 mma rows softcap d={d}")
    assert np.all(O[2] == 0) and np.all(L[2] == -np.inf)


# (d, n_head, n_head_kv, n_q): more than 8 rows per KV head over a segment: row groups of 16 (the
# last one ragged), one workgroup per (row group, split, head group)
ROW_GROUPS = [(64, 64, 8, 2), (64, 40, 8, 5), (256, 48, 4, 3), (512, 20, 2, 3), (576, 16, 1, 2), (576, 40, 2, 1)]


@pytest.mark.parametrize("d,n_head,n_head_kv,n_q", ROW_GROUPS)
def test_row_groups(run, d, n_head, n_head_kv, n_q):
    w = workload(2, d, scale_down=64, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)  # n_kv 2048
    mask = gen.random_mask_f16(np.random.default_rng(d + n_head), n_q, w["n_kv"], p_hidden=0.2)
    step(f"f16 mma row groups d={d} heads {n_head}/{n_head_kv} n_q {n_q} ({n_q * n_head // n_head_kv} rows per KV head)")
    O, L = run.decode(w, wc=1300, tile_kv=400, tail="host", mask=mask)
    assert run.ctx.stats()["kernel_variant"] == MMA16
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"f16 mma row groups d={d} {n_head}/{n_head_kv} n_q {n_q}")


@pytest.mark.parametrize("d", [64, 256, 512, 576])
def test_prefill_row_groups_causal(run, d):
    """A prefill chunk of 24 queries of 4 heads per KV head (96 rows: six row groups) at the end
    of a window + lifted tail, causal, with a mask hiding some keys and one query seeing none
    (at 64 the prefill kernel takes the chunk)."""
    w = workload(5, d, scale_down=64, n_head=32, n_head_kv=8)  # n_kv 1664
    n_q = 24
    w["q"] = w["q"][:, -n_q:]
    q_pos0 = w["n_kv"] - n_q
    mask = gen.random_mask_f16(np.random.default_rng(d), n_q, w["n_kv"], p_hidden=0.1)
    mask[5, :] = -np.inf
    step(f"f16 mma prefill row groups d={d}: {n_q} queries, causal, masked")
    O, L = run.decode(w, wc=1000, tile_kv=256, tail="host", mask=mask, prefill=True, q_pos0=q_pos0)
    assert run.ctx.stats()["kernel_variant"] == (1 if d == 64 else MMA16)
    full = np.where(oracle.causal_mask(n_q, w["n_kv"], q_pos0) == -np.inf, -np.inf, mask.astype(np.float64))
    Oref, Lref = oracle_decode(w, mask=full)
    assert_close(O, L, Oref, Lref, what=f"f16 prefill row groups d={d}")
    assert np.all(O[5] == 0) and np.all(L[5] == -np.inf)
