"""GPU parity of rkv_attn_prefill at head dim 64 (dk = dv = 64, more than 8 rows per KV head),
which runs the matrix-core prefill kernel instantiated for 64 (two 32-value parts per row, two
output tiles), against the fp64 oracle: causal chunks over a window + lifted tail, the four type
pairs, masks with empty rows, the soft-cap, ragged query tiles and key counts, outlier keys,
the head-major layout, and the full-size 512-query chunk on sampled KV heads (opencoti-llamafile
patch 0070-rolling-kv: the segment partials and their combine; the pages' prefill chunk)."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, oracle_decode, step

pytestmark = pytest.mark.gpu

PREFILL_MFMA = 1
D = 64


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_softcap(0.0)


def chunk(num=5, n_kv=1664, n_q=160, wc=1024, tile=512, **over):
    """A prefill chunk at head dim 64: the chunk's n_q queries are the last n_q positions."""
    base = gen.WORKLOADS[num]
    sd = max(1, base["n_kv"] // n_kv)
    w = gen.make_workload(num, scale_down=sd, n_q=n_q, d=D, dv=D, **over)
    w["wc"], w["tile_kv"] = min(wc, w["n_kv"]), tile
    w["q_pos0"] = w["n_kv"] - n_q
    return w


def causal_ref(w, q_pos0=None, mask=None, softcap=0.0):
    q_pos0 = w["q_pos0"] if q_pos0 is None else q_pos0
    n_q = w["q"].shape[1]
    m = oracle.causal_mask(n_q, w["n_kv"], q_pos0) if q_pos0 >= 0 else np.zeros((n_q, w["n_kv"]))
    if mask is not None:
        m = m + np.asarray(mask, dtype=np.float64)
    return oracle_decode(w, mask=m, softcap=softcap)


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_F16, gen.TYPE_F16),
                                   (gen.TYPE_Q8_0, gen.TYPE_F16), (gen.TYPE_F16, gen.TYPE_Q4_0)])
def test_causal_chunk_window_and_tail_tiles(run, kt, vt):
    # 40/8 heads, 160 queries (800 rows per KV head: 3 full row tiles + a ragged one), window
    # 1024 + host tail 640 in tiles 512 + 128
    w = chunk(k_type=kt, v_type=vt)
    step(f"prefill d64 k={kt} v={vt} n_q=160 n_kv={w['n_kv']} wc=1024 tile=512, causal")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    st = run.ctx.stats()
    assert st["kernel_variant"] == PREFILL_MFMA and st["n_tail_tiles"] == 2
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what=f"d64 causal {kt}/{vt}")


@pytest.mark.parametrize("tile", [31, 100, 4096])
def test_tile_sweep_ragged(run, tile):
    w = chunk(n_kv=1664, n_q=40, wc=1333, tile=tile)
    step(f"prefill d64 q8q4 wc=1333 tile={tile}")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what=f"d64 tile {tile}")


def test_mask_only_with_empty_rows(run):
    w = chunk(n_kv=1664, n_q=24, wc=1000, tile=400, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16)
    rng = np.random.default_rng(64)
    mask = gen.random_mask_f16(rng, 24, w["n_kv"], p_hidden=0.35)
    mask[5, :] = -np.inf  # query 5 sees nothing
    mask[17, 1000:] = -np.inf  # query 17 sees the window only
    step("prefill d64 f16 mask only (q_pos0=-1), empty row")
    O, L = run.decode(w, prefill=True, q_pos0=-1, tail="host", mask=mask)
    assert run.ctx.stats()["kernel_variant"] == PREFILL_MFMA
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="d64 mask")
    assert np.all(O[5] == 0) and np.all(L[5] == -np.inf)


def test_causal_plus_mask_chunk_in_the_middle(run):
    """q_pos0 inside the window: later keys and whole tail tiles are hidden, and a mask on top."""
    w = chunk(n_kv=1664, n_q=64, wc=1024, tile=256)
    mask = gen.random_mask_f16(np.random.default_rng(65), 64, w["n_kv"], p_hidden=0.2)
    step("prefill d64 q8q4 q_pos0=500 + mask")
    O, L = run.decode(w, prefill=True, q_pos0=500, tail="host", mask=mask)
    Oref, Lref = causal_ref(w, q_pos0=500, mask=mask)
    assert_close(O, L, Oref, Lref, what="d64 middle + mask")


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_F16, gen.TYPE_F16)])
def test_softcap(run, kt, vt):
    w = chunk(n_kv=1664, n_q=48, wc=900, tile=333, k_type=kt, v_type=vt)
    run.ctx.set_softcap(2.0)
    try:
        step(f"prefill d64 soft-cap 2.0 k={kt} v={vt}")
        O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = causal_ref(w, softcap=2.0)
    assert_close(O, L, Oref, Lref, what="d64 softcap")


@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(8, 8, 9), (8, 2, 3), (6, 2, 50), (7, 1, 40), (64, 1, 9)])
def test_group_shapes(run, n_head, n_head_kv, n_q):
    w = chunk(n_kv=1664, n_q=n_q, wc=1200, tile=300, n_head=n_head, n_head_kv=n_head_kv)
    step(f"prefill d64 gqa shape {n_head}/{n_head_kv} n_q={n_q}")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    assert run.ctx.stats()["kernel_variant"] == PREFILL_MFMA
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="d64 gqa")


def test_outlier_keys_exact_k(run):
    """Every 17th key scaled x30: q8_0 K enters the matrix cores as two exact binary16 parts."""
    rng = gen.rng_for(97)
    n_q, n_kv = 64, 1600
    q, k, v = gen.draw_qkv(rng, 40, n_q, 8, n_kv, d=D, dv=D, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0,
                           outlier_every=17)
    w = dict(n_head=40, n_head_kv=8, q=q, k=k, v=v, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0,
             scale=1 / np.sqrt(D), n_kv=n_kv, wc=1000, tile_kv=300, q_pos0=n_kv - n_q, dv=D)
    step("prefill d64 outlier keys x30 every 17th")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="d64 outliers")


def test_head_major_layout(run):
    w = chunk(n_kv=1664, n_q=32, wc=1024, tile=512)
    step("prefill d64 q8q4 head-major layout, device tail")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="device", layout="head")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="d64 head-major")


def test_eight_rows_stay_on_the_decode_kernels(run):
    """8 rows per KV head (2 queries of 4 heads) at head dim 64 keep the decode kernels."""
    w = chunk(n_kv=1664, n_q=2, wc=1024, tile=512, n_head=32, n_head_kv=8)
    step("prefill d64 8 rows per KV head")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    assert run.ctx.stats()["kernel_variant"] != PREFILL_MFMA
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="d64 8 rows")


def test_full_size_chunk_sampled_heads(run):
    """The 512-query chunk against n_kv=106496 (window 65536 + host tail in tiles of 32768) at
    head dim 64, in the launch configuration the benchmark times at that head dim; the oracle
    checks all 512 queries of every query head of KV heads 2 and 7 over all keys."""
    w = gen.make_workload(5, d=D, dv=D)
    step("prefill d64 full size n_q=512 n_kv=106496 wc=65536 tile=32768 host tail")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    assert run.ctx.stats()["kernel_variant"] == PREFILL_MFMA
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    gqa = w["n_head"] // w["n_head_kv"]
    mask = oracle.causal_mask(512, w["n_kv"], w["q_pos0"])
    for g in (2, 7):
        kv = oracle.kv_values(w["k_type"], w["k"][:, g:g + 1])
        vv = oracle.kv_values(w["v_type"], w["v"][:, g:g + 1])
        for i0 in range(0, 512, 64):
            qi = np.arange(i0, i0 + 64)
            qv = oracle.q_values(w["q"][g * gqa:(g + 1) * gqa][:, qi])
            Oref, Lref = oracle.attention(qv, kv, vv, w["scale"], mask[qi])
            assert_close(O[qi][:, g * gqa:(g + 1) * gqa], L[qi][:, g * gqa:(g + 1) * gqa], Oref, Lref,
                         what=f"d64 full size head group {g} queries {i0}..{i0 + 63}")


TYPES = [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
         (gen.TYPE_F16, gen.TYPE_Q4_0)]


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_d64(run, seed):
    """Random heads (more than 8 rows per KV head), query and key counts, window + tail splits,
    types, layouts, masks and soft-caps at head dim 64."""
    rng = np.random.default_rng(6400 + seed)
    n_head_kv = int(rng.choice([1, 2, 8]))
    gqa = int(rng.choice([1, 4, 5, 8]))
    n_q = int(rng.integers(max(2, 9 // gqa + 1), 300))
    n_kv = int(rng.integers(n_q, 2200))
    kt, vt = TYPES[int(rng.integers(0, 4))]
    wc = int(rng.integers(0, n_kv + 1))
    tile = int(rng.integers(1, 1200))
    layout = str(rng.choice(["cell", "head"]))
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_kv, d=D, dv=D, k_type=kt, v_type=vt)
    w = dict(n_head=n_head_kv * gqa, n_head_kv=n_head_kv, q=q, k=k, v=v, k_type=kt, v_type=vt, dv=D,
             scale=1 / np.sqrt(D), n_kv=n_kv, wc=wc, tile_kv=tile)
    q_pos0 = n_kv - n_q if rng.random() < 0.7 else int(rng.integers(0, n_kv - n_q + 1))
    mask = gen.random_mask_f16(rng, n_q, n_kv, p_hidden=0.2) if rng.random() < 0.3 else None
    cap = float(rng.uniform(0.5, 5.0)) if rng.random() < 0.35 else 0.0
    step(f"random prefill d64 seed {seed}: heads {n_head_kv}x{gqa} n_q {n_q} n_kv {n_kv} wc {wc} tile {tile} "
         f"types {kt}/{vt} layout {layout} q_pos0 {q_pos0} mask {mask is not None} softcap {cap:.3f}")
    run.ctx.set_softcap(cap)
    try:
        O, L = run.decode(w, prefill=True, q_pos0=q_pos0, tail="host" if wc < n_kv else None, mask=mask,
                          layout=layout)
        assert run.ctx.stats()["kernel_variant"] == PREFILL_MFMA
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = causal_ref(w, q_pos0=q_pos0, mask=mask, softcap=cap)
    assert_close(O, L, Oref, Lref, what=f"random prefill d64 {seed}")

