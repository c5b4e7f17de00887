"""Randomised GPU parity sweep: seeded random shapes, types, layouts, splits, tails, lift modes,
masks, row lists (with holes and entries past the pool), logit soft-caps and head dims through every entry point, each case against the fp64 oracle.  The cases are small
(the oracle runs them in well under a second) and cover combinations the targeted tests do
not enumerate: every kernel family is reached (vector, matrix-core q8_0/q4_0, matrix-core
binary16 window/tail/rows, prefill), with ragged lengths throughout."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, oracle_rows, step

pytestmark = pytest.mark.gpu

TYPES = [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
         (gen.TYPE_F16, gen.TYPE_Q4_0)]


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_softcap(0.0)


def draw_softcap(seed: int) -> float:
    """A logit soft-cap for about a third of the cases, drawn apart from the case's own draws."""
    rng = np.random.default_rng(5000 + seed)
    return float(rng.uniform(0.5, 5.0)) if rng.random() < 0.35 else 0.0


@pytest.mark.parametrize("seed", range(24))
def test_random_decode(run, seed):
    rng = np.random.default_rng(1000 + seed)
    n_head_kv = int(rng.choice([1, 2, 4, 8, 8, 16]))
    gqa = int(rng.choice([1, 2, 3, 4, 5, 8]))
    n_q = int(rng.choice([1, 1, 2]))
    n_kv = int(rng.integers(1, 2500))
    kt, vt = TYPES[int(rng.integers(0, 4))]
    tail = str(rng.choice(["host", "device", "none"]))
    wc = n_kv if tail == "none" else int(rng.integers(0, n_kv + 1))
    if wc == n_kv:
        tail = "none"
    tile = int(rng.integers(1, 1500))
    layout = str(rng.choice(["cell", "cell", "head"]))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, k_type=kt, v_type=vt)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=kt, v_type=vt,
             scale=1 / np.sqrt(128), n_kv=n_kv, wc=wc, tile_kv=tile)
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.3) if rng.random() < 0.5 else None
    step(f"random decode seed {seed}: heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} tile {tile} "
         f"types {kt}/{vt} tail {tail} layout {layout} mask {mask is not None}")
    cap = draw_softcap(seed)
    run.ctx.set_softcap(cap)
    lift = int(np.random.default_rng(7000 + seed).choice([run.rkv.RKV_LIFT_AUTO, run.rkv.RKV_LIFT_BULK,
                                                          run.rkv.RKV_LIFT_KERNEL]))
    run.ctx.set_lift_mode(lift)
    step(f"  softcap {cap:.3f} lift mode {lift}")
    try:
        O, L = run.decode(w, tail=None if tail == "none" else tail, mask=mask, layout=layout)
    finally:
        run.ctx.set_lift_mode(run.rkv.RKV_LIFT_AUTO)
    Oref, Lref = oracle_decode(w, mask=mask, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random decode {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_rows(run, seed):
    rng = np.random.default_rng(2000 + seed)
    n_head_kv = int(rng.choice([1, 2, 8, 8, 16]))
    gqa = int(rng.choice([1, 2, 4, 8]))
    n_q = 1 if gqa == 8 else int(rng.choice([1, 2]))
    n_seq = int(rng.integers(1, 5))
    n_pool = int(rng.integers(50, 2000))
    kt, vt = TYPES[0] if rng.random() < 0.6 else TYPES[int(rng.integers(1, 4))]
    lengths = tuple(int(x) for x in rng.integers(0, 1200, size=n_seq))
    n_kv = max(1, max(lengths))
    rows = gen.rows_lists(rng, n_pool, lengths, n_kv, shuffle=bool(rng.random() < 0.5))
    if rng.random() < 0.5:  # holes inside the lists
        rows[rng.random(rows.shape) < 0.2] = -1
    q = gen.draw_normal(rng, (n_seq, n_head_kv * gqa, n_q, 128)).astype(np.float16)
    k = gen.pack(kt, gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    v = gen.pack(vt, gen.draw_normal(rng, (n_pool, n_head_kv, 128)))
    mask = None
    if rng.random() < 0.5:
        mask = np.stack([gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.2) for _ in range(n_seq)])[:, None]
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=mask, k_type=kt, v_type=vt, scale=1 / np.sqrt(128))
    step(f"random rows seed {seed}: heads {n_head_kv}x{gqa} n_q {n_q} seqs {lengths} pool {n_pool} "
         f"types {kt}/{vt} mask {mask is not None}")
    cap = draw_softcap(100 + seed)
    run.ctx.set_softcap(cap)
    step(f"  softcap {cap:.3f}")
    O, L = run.rows(w)  # the mask (or None) travels in w
    Oref, Lref = oracle_rows(w, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random rows {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_random_prefill(run, seed):
    rng = np.random.default_rng(3000 + seed)
    n_head_kv = int(rng.choice([1, 2, 8]))
    gqa = int(rng.choice([1, 4, 5]))
    n_q = int(rng.integers(2, 200))
    n_kv = int(rng.integers(n_q, 2200))
    kt, vt = TYPES[int(rng.integers(0, 4))]
    wc = int(rng.integers(0, n_kv + 1))
    tile = int(rng.integers(1, 1200))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, k_type=kt, v_type=vt)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=kt, v_type=vt,
             scale=1 / np.sqrt(128), n_kv=n_kv, wc=wc, tile_kv=tile)
    q_pos0 = n_kv - n_q if rng.random() < 0.7 else int(rng.integers(0, n_kv - n_q + 1))
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.2) if rng.random() < 0.3 else None
    step(f"random prefill seed {seed}: heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} tile {tile} "
         f"types {kt}/{vt} q_pos0 {q_pos0} mask {mask is not None}")
    cap = draw_softcap(200 + seed)
    run.ctx.set_softcap(cap)
    step(f"  softcap {cap:.3f}")
    O, L = run.decode(w, prefill=True, q_pos0=q_pos0, tail="host" if wc < n_kv else None, mask=mask)
    m = oracle.causal_mask(n_q, n_kv, q_pos0)
    if mask is not None:
        m = m + np.asarray(mask, dtype=np.float64)
    Oref, Lref = oracle_decode(w, mask=m, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random prefill {seed}")


@pytest.mark.parametrize("seed", range(12))
def test_random_host_tail(run, seed):
    """Decode with the tail partial on the host cores: random shapes, types, layouts, window
    sizes, masks, soft-caps, thread counts, pinned or pageable tails."""
    rng = np.random.default_rng(4000 + seed)
    n_head_kv = int(rng.choice([1, 2, 4, 8]))
    gqa = int(rng.choice([1, 2, 4, 5, 8]))
    n_q = 1 if gqa > 4 else int(rng.choice([1, 2]))
    n_kv = int(rng.integers(2, 2500))
    kt, vt = TYPES[int(rng.integers(0, 4))]
    wc = int(rng.integers(0, n_kv))
    layout = str(rng.choice(["cell", "head"]))
    tail = str(rng.choice(["host", "pageable"]))
    threads = int(rng.integers(1, 17))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, k_type=kt, v_type=vt)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=kt, v_type=vt,
             scale=1 / np.sqrt(128), n_kv=n_kv, wc=wc, tile_kv=int(rng.integers(1, 2000)))
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.3) if rng.random() < 0.5 else None
    cap = draw_softcap(300 + seed)
    step(f"random host tail seed {seed}: heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} types {kt}/{vt} "
         f"layout {layout} tail {tail} threads {threads} mask {mask is not None} softcap {cap:.3f}")
    run.ctx.set_softcap(cap)
    run.ctx.set_tail_mode(run.rkv.RKV_TAIL_HOST, threads)
    try:
        O, L = run.decode(w, tail=tail, mask=mask, layout=layout)
        assert run.ctx.stats()["tail_host"] == 1
    finally:
        run.ctx.set_tail_mode(run.rkv.RKV_TAIL_LIFT)
    Oref, Lref = oracle_decode(w, mask=mask, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random host tail {seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_head_dims(run, seed):
    """Head dims 64, 256, 512 and 576/512 through the window + tail split: random heads (up to
    48 query rows per KV head: row groups on the matrix-core kernel, groups of 8 on the vector
    kernel), lengths, splits, types, layouts, tails, lift engines, masks and soft-caps."""
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([64, 256, 512, 576]))
    dv = 512 if d == 576 else d
    n_head_kv = int(rng.choice([1, 2, 4, 8]))
    n_q = int(rng.choice([1, 1, 2, 3]))
    gqa = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    n_kv = int(rng.integers(1, 2500))
    kt, vt = TYPES[1] if rng.random() < 0.5 else TYPES[int(rng.integers(0, 4))]
    tail = str(rng.choice(["host", "device", "none"]))
    wc = n_kv if tail == "none" else int(rng.integers(0, n_kv + 1))
    if wc == n_kv:
        tail = "none"
    tile = int(rng.integers(1, 1500))
    layout = str(rng.choice(["cell", "head"]))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, d=d, dv=dv, k_type=kt, v_type=vt)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=kt, v_type=vt, d=d, dv=dv,
             scale=1 / np.sqrt(d), n_kv=n_kv, wc=wc, tile_kv=tile)
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.3) if rng.random() < 0.5 else None
    cap = draw_softcap(100 + seed)
    lift = int(rng.choice([run.rkv.RKV_LIFT_BULK, run.rkv.RKV_LIFT_KERNEL]))
    step(f"random head-dim decode seed {seed}: d {d}/{dv} heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} "
         f"tile {tile} types {kt}/{vt} tail {tail} layout {layout} mask {mask is not None} softcap {cap:.3f} "
         f"lift {lift}")
    run.ctx.set_softcap(cap)
    run.ctx.set_lift_mode(lift)
    try:
        O, L = run.decode(w, tail=None if tail == "none" else tail, mask=mask, layout=layout)
    finally:
        run.ctx.set_lift_mode(run.rkv.RKV_LIFT_AUTO)
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, mask=mask, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random head-dim decode {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_rows_head_dims(run, seed):
    """Row lists at every head dim: random pools (q8_0/q4_0 on the matrix-core kernel, binary16
    on the vector or persistent binary16 kernel), sequences, list lengths, shuffled order,
    -1 holes, entries past the pool (no key: the oracle takes them as -1), up to 32 query rows
    per KV head away from head dim 128, masks and soft-caps."""
    rng = np.random.default_rng(11000 + seed)
    d = int(rng.choice([64, 128, 256, 512, 576]))
    dv = 512 if d == 576 else d
    n_head_kv = int(rng.choice([1, 2, 4, 8]))
    n_q = int(rng.choice([1, 1, 2]))
    gqas = (1, 2, 4, 8) if d == 128 else (1, 2, 4, 5, 8, 16)
    gqa = int(rng.choice([g for g in gqas if d != 128 or g * n_q <= 8]))
    n_seq = int(rng.integers(1, 4))
    n_pool = int(rng.integers(50, 1500))
    kt, vt = TYPES[1] if rng.random() < 0.7 else TYPES[0]
    lengths = tuple(int(x) for x in rng.integers(0, 1100, size=n_seq))
    n_kv = max(1, max(lengths))
    rows = gen.rows_lists(rng, n_pool, lengths, n_kv, shuffle=bool(rng.random() < 0.5))
    holes = (rng.random(rows.shape) < 0.1) & (rows >= 0)
    rows[holes] = -1
    past = (rng.random(rows.shape) < 0.03) & (rows >= 0)
    rows[past] = n_pool + rng.integers(0, 5000, int(past.sum()))
    q = gen.draw_normal(rng, (n_seq, n_head_kv * gqa, n_q, d)).astype(np.float16)
    k = gen.pack(kt, gen.draw_normal(rng, (n_pool, n_head_kv, d)))
    v = gen.pack(vt, gen.draw_normal(rng, (n_pool, n_head_kv, dv)))
    mask = None
    if rng.random() < 0.5:
        mask = np.where(rng.random((n_seq, 1, n_q, n_kv)) < 0.2, -np.inf, 0.0).astype(np.float16)
    w = dict(q=q, k=k, v=v, kv_rows=rows, mask=mask, k_type=kt, v_type=vt, n_head=n_head_kv * gqa,
             n_head_kv=n_head_kv, scale=1 / np.sqrt(d), d=d, dv=dv)
    cap = draw_softcap(300 + seed)
    step(f"random rows seed {seed}: d {d}/{dv} heads {n_head_kv}x{gqa} n_q {n_q} seqs {lengths} pool {n_pool} "
         f"types {kt}/{vt} mask {mask is not None} softcap {cap:.3f}")
    run.ctx.set_softcap(cap)
    try:
        O, L = run.rows(w)
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_rows(w, rows=np.where(rows < n_pool, rows, -1), softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random rows {seed}")


@pytest.mark.parametrize("seed", range(20))
def test_random_binary16_cell_groups(run, seed):
    """The persistent binary16 matrix-core kernel at head dims 64, 128, 256, 512 and 576 / 512:
    random head groups (KV heads a multiple of the group of 8, 8, 4, 2 or 1), up to 8 rows per KV head,
    lengths, window + tail splits (lifted or on the device), masks, a small causal prefill in a
    quarter of the cases, and soft-caps; every case but prefill at 128 must run on that kernel."""
    rng = np.random.default_rng(13000 + seed)
    d = int(rng.choice([64, 128, 256, 512, 576]))
    dv = 512 if d == 576 else d
    hw = {64: 8, 128: 8, 256: 4, 512: 2, 576: 1}[d]
    n_head_kv = hw * int(rng.choice([1, 1, 2]))
    n_q = int(rng.choice([1, 1, 2]))
    gqa = int(rng.choice([g for g in (1, 2, 3, 4, 5, 8) if g * n_q <= 8]))
    n_kv = int(rng.integers(1, 3000))
    tail = str(rng.choice(["host", "device", "none"]))
    wc = n_kv if tail == "none" else int(rng.integers(0, n_kv + 1))
    if wc == n_kv:
        tail = "none"
    tile = int(rng.integers(1, 1500))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, d=d, dv=dv, k_type=gen.TYPE_F16,
                           v_type=gen.TYPE_F16)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=gen.TYPE_F16,
             v_type=gen.TYPE_F16, d=d, dv=dv, scale=1 / np.sqrt(d), n_kv=n_kv, wc=wc, tile_kv=tile)
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.3) if rng.random() < 0.5 else None
    prefill = n_q > 1 and rng.random() < 0.5
    q_pos0 = int(rng.integers(0, n_kv)) if prefill else -1
    cap = draw_softcap(700 + seed)
    step(f"random binary16 cell groups seed {seed}: d {d} heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} "
         f"tile {tile} tail {tail} mask {mask is not None} prefill {prefill} q_pos0 {q_pos0} softcap {cap:.3f}")
    run.ctx.set_softcap(cap)
    try:
        O, L = run.decode(w, tail=None if tail == "none" else tail, mask=mask, prefill=prefill, q_pos0=q_pos0)
        # (prefill at 128 runs on the matrix-core prefill kernel)
        assert run.ctx.stats()["kernel_variant"] == (1 if prefill and d == 128 else 4)
    finally:
        run.ctx.set_softcap(0.0)
    full = mask if mask is not None else np.zeros((n_q, n_kv), np.float16)
    if prefill:
        full = np.where(oracle.causal_mask(n_q, n_kv, q_pos0) == -np.inf, -np.inf, full.astype(np.float64))
    Oref, Lref = oracle_decode(w, mask=full if (prefill or mask is not None) else None, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random binary16 cell groups {seed}")
