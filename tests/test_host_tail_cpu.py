"""The tail partial on the host cores (rkv_tail_partial_host, the computation behind
RKV_TAIL_HOST) against the fp64 oracle.  Pure host code: runs without a GPU.

The partial (M, S, VKQ) of a segment is compared after normalisation (O = VKQ / S,
LSE = M + ln S) at the spec tolerances, alone and merged with oracle partials of the other
segments of a split (the partition invariance the merge relies on)."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import assert_close

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rkv():
    import os
    import tiered_kv_cache_split_amd as m
    from tiered_kv_cache_split_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("librkv.so is not built (run __graft_entry__.build())")
    return m


def host_cache(cache, layout):
    """Cell-major bytes (n_cells, n_head_kv, row) as a CPU tensor in the requested layout."""
    if layout == "head":
        cache = np.ascontiguousarray(np.transpose(cache, (1, 0, 2)))
    return torch.from_numpy(np.ascontiguousarray(cache))


def run_host(rkv, q, k, v, k_type, v_type, mask=None, kv_pos0=0, q_pos0=-1, scale=1 / np.sqrt(128),
             softcap=0.0, layout="cell", n_threads=0):
    n_head, n_q, _ = q.shape
    qt = torch.from_numpy(np.ascontiguousarray(q))
    kt, vt = host_cache(k, layout), host_cache(v, layout)
    mt = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    dv = gen.values_per_row(v_type, v.shape[-1])
    part = torch.full((n_q, n_head, 2 + dv), float("nan"), dtype=torch.float32)
    rkv.tail_partial_host(rkv.q_desc(qt), rkv.kv_desc(kt, k_type, layout), rkv.kv_desc(vt, v_type, layout),
                          rkv.mask_desc(mt), kv_pos0, q_pos0, scale, part, softcap=softcap, n_threads=n_threads)
    p = part.numpy().astype(np.float64)
    return p[..., 0], p[..., 1], p[..., 2:]


def oracle_partial(q, k, v, k_type, v_type, mask_cols=None, scale=1 / np.sqrt(128), softcap=0.0):
    return oracle.partial(oracle.q_values(q), oracle.kv_values(k_type, k), oracle.kv_values(v_type, v), scale,
                          mask_cols, softcap)


def check_partial(host, ref, what):
    O, L = oracle.merge([host])
    Oref, Lref = oracle.merge([ref])
    assert_close(O, L, Oref, Lref, what=what)
    fin = np.isfinite(ref[0])
    assert np.array_equal(np.isfinite(host[0]), fin), what
    assert np.all(host[1][~fin] == 0) and np.all(host[2][~fin] == 0), what
    if fin.any():
        assert np.abs(host[0][fin] - ref[0][fin]).max() <= 1e-3, what


@pytest.mark.parametrize("layout", ["cell", "head"])
def test_q8q4_matches_oracle(rkv, layout):
    rng = np.random.default_rng(1101)
    q, k, v = gen.draw_qkv(rng, 40, 1, 8, 5003, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    host = run_host(rkv, q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0, kv_pos0=131072, layout=layout)
    check_partial(host, oracle_partial(q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0), f"q8q4 {layout}")


def test_f16_mask_at_global_columns(rkv):
    rng = np.random.default_rng(1102)
    n_q, n_cells, kv_pos0 = 3, 2500, 777
    q, k, v = gen.draw_qkv(rng, 8, n_q, 2, n_cells)
    mask = gen.random_mask_f16(rng, n_q, kv_pos0 + n_cells + 5)
    host = run_host(rkv, q, k, v, gen.TYPE_F16, gen.TYPE_F16, mask=mask, kv_pos0=kv_pos0, layout="head")
    ref = oracle_partial(q, k, v, gen.TYPE_F16, gen.TYPE_F16, mask[:, kv_pos0:kv_pos0 + n_cells])
    check_partial(host, ref, "f16 mask")


def test_causal_positions(rkv):
    rng = np.random.default_rng(1103)
    n_q, n_cells, kv_pos0, q_pos0 = 5, 300, 100, 380
    q, k, v = gen.draw_qkv(rng, 4, n_q, 2, n_cells, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_F16)
    host = run_host(rkv, q, k, v, gen.TYPE_Q8_0, gen.TYPE_F16, kv_pos0=kv_pos0, q_pos0=q_pos0)
    cm = oracle.causal_mask(n_q, kv_pos0 + n_cells, q_pos0)[:, kv_pos0:]
    check_partial(host, oracle_partial(q, k, v, gen.TYPE_Q8_0, gen.TYPE_F16, cm), "causal")


def test_softcap_with_outlier_keys(rkv):
    rng = np.random.default_rng(1104)
    q, k, v = gen.draw_qkv(rng, 8, 1, 2, 3000, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0, outlier_every=17)
    for cap in (0.0, 5.0):
        host = run_host(rkv, q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0, softcap=cap)
        ref = oracle_partial(q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0, softcap=cap)
        check_partial(host, ref, f"outliers cap {cap}")


def test_split_merges_with_device_segments(rkv):
    """Window and first tail tile from the oracle, last tile from the host: the merge equals
    unsplit attention."""
    rng = np.random.default_rng(1105)
    n_kv, wc = 6000, 3500
    q, k, v = gen.draw_qkv(rng, 40, 1, 8, n_kv, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    qv, kv_, vv = oracle.q_values(q), oracle.kv_values(gen.TYPE_Q8_0, k), oracle.kv_values(gen.TYPE_Q4_0, v)
    s = 1 / np.sqrt(128)
    parts = [oracle.partial(qv, kv_[:, :wc], vv[:, :wc], s), oracle.partial(qv, kv_[:, wc:5000], vv[:, wc:5000], s),
             run_host(rkv, q, k[5000:], v[5000:], gen.TYPE_Q8_0, gen.TYPE_Q4_0, kv_pos0=5000)]
    O, L = oracle.merge(parts)
    Oref, Lref = oracle.attention(qv, kv_, vv, s)
    assert_close(O, L, Oref, Lref, what="split merge")


def test_empty_rows_and_empty_segment(rkv):
    rng = np.random.default_rng(1106)
    q, k, v = gen.draw_qkv(rng, 4, 2, 2, 100)
    mask = np.zeros((2, 100), dtype=np.float16)
    mask[1, :] = -np.inf  # query 1 sees nothing
    M, S, V = run_host(rkv, q, k, v, gen.TYPE_F16, gen.TYPE_F16, mask=mask)
    assert np.all(M[1] == -np.inf) and np.all(S[1] == 0) and np.all(V[1] == 0)
    assert np.all(np.isfinite(M[0]))
    M, S, V = run_host(rkv, q, k[:0], v[:0], gen.TYPE_F16, gen.TYPE_F16)
    assert np.all(M == -np.inf) and np.all(S == 0) and np.all(V == 0)


def test_thread_counts(rkv):
    rng = np.random.default_rng(1107)
    q, k, v = gen.draw_qkv(rng, 40, 1, 8, 4096, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    ref = oracle_partial(q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0)
    for n in (1, 3, 16):
        check_partial(run_host(rkv, q, k, v, gen.TYPE_Q8_0, gen.TYPE_Q4_0, n_threads=n), ref, f"{n} threads")


def test_argument_errors(rkv):
    from tiered_kv_cache_split_amd import _lib
    rng = np.random.default_rng(1108)
    q, k, v = gen.draw_qkv(rng, 4, 1, 2, 64)
    qt, kt, vt = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    part = torch.zeros((1, 4, 130), dtype=torch.float32)
    qd, kd, vd = rkv.q_desc(qt), rkv.kv_desc(kt, gen.TYPE_F16), rkv.kv_desc(vt, gen.TYPE_F16)
    small = torch.zeros((1, 32), dtype=torch.float16)
    cases = [
        (dict(mask=rkv.mask_desc(small)), _lib.RKV_ERR_ARG),          # mask narrower than the segment
        (dict(partial=None), _lib.RKV_ERR_ARG),
        (dict(n_threads=300), _lib.RKV_ERR_ARG),
        (dict(kv_pos0=-1), _lib.RKV_ERR_ARG),
        (dict(softcap=-1.0), _lib.RKV_ERR_ARG),
        (dict(v=rkv.kv_desc(vt, gen.TYPE_F16, "cell")), None),
    ]
    lib = _lib.load()
    import ctypes
    for over, want in cases:
        a = dict(q=qd, k=kd, v=vd, mask=None, kv_pos0=0, q_pos0=-1, scale=0.1, softcap=0.0, partial=part,
                 n_threads=0)
        a.update(over)
        st = lib.rkv_tail_partial_host(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                       None if a["mask"] is None else ctypes.byref(a["mask"]), a["kv_pos0"],
                                       a["q_pos0"], a["scale"], a["softcap"],
                                       None if a["partial"] is None else a["partial"].data_ptr(), a["n_threads"])
        if want is None:
            assert st == _lib.RKV_OK, lib.rkv_last_error()
        else:
            assert st == want, (over, st)
    bad = rkv.kv_desc(kt, gen.TYPE_F16)
    bad.type = _lib.RKV_TYPE_F32
    assert lib.rkv_tail_partial_host(ctypes.byref(qd), ctypes.byref(bad), ctypes.byref(vd), None, 0, -1, 0.1, 0.0,
                                     part.data_ptr(), 0) == _lib.RKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(rkv, seed):
    """Random heads (gqa up to 16: several row groups of a KV head), queries, lengths, types,
    layouts, masks, causal positions, soft-caps and thread counts."""
    rng = np.random.default_rng(6000 + seed)
    n_head_kv = int(rng.choice([1, 2, 3, 8]))
    gqa = int(rng.choice([1, 3, 5, 8, 12, 16]))
    n_q = int(rng.integers(1, 5))
    n_cells = int(rng.integers(0, 1500))
    kv_pos0 = int(rng.integers(0, 3000))
    kt, vt = [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
              (gen.TYPE_F16, gen.TYPE_Q4_0)][int(rng.integers(0, 4))]
    q, k, v = gen.draw_qkv(rng, n_head_kv * gqa, n_q, n_head_kv, n_cells, k_type=kt, v_type=vt)
    mask = gen.random_mask_f16(rng, n_q, kv_pos0 + n_cells, p_hidden=0.3) if rng.random() < 0.5 else None
    q_pos0 = int(rng.integers(kv_pos0 - 5, kv_pos0 + n_cells + 5)) if rng.random() < 0.4 else -1
    q_pos0 = max(q_pos0, -1)
    cap = float(rng.uniform(0.5, 5.0)) if rng.random() < 0.3 else 0.0
    layout = str(rng.choice(["cell", "head"]))
    host = run_host(rkv, q, k, v, kt, vt, mask=mask, kv_pos0=kv_pos0, q_pos0=q_pos0, softcap=cap, layout=layout,
                    n_threads=int(rng.integers(1, 9)))
    cols = np.zeros((n_q, n_cells))
    if mask is not None:
        cols = cols + np.asarray(mask[:, kv_pos0:kv_pos0 + n_cells], dtype=np.float64)
    if q_pos0 >= 0:
        cols = cols + oracle.causal_mask(n_q, kv_pos0 + n_cells, q_pos0)[:, kv_pos0:]
    ref = oracle_partial(q, k, v, kt, vt, cols, softcap=cap)
    check_partial(host, ref, f"random {seed}")


def test_choose_tail_mode(rkv):
    """The tactic with the shorter tail time: host partial only when the host cores read the
    tail faster than the link lifts it; the lift wins ties, an empty tail and bad rates fail."""
    from tiered_kv_cache_split_amd import _lib
    tb = 218103808
    assert rkv.choose_tail_mode(tb, 57.0, 48.9) == rkv.RKV_TAIL_LIFT      # the MI355X machine measured here
    assert rkv.choose_tail_mode(tb, 12.0, 48.9) == rkv.RKV_TAIL_HOST      # a slow link (UVA-class rates)
    assert rkv.choose_tail_mode(tb, 30.0, 30.0) == rkv.RKV_TAIL_LIFT      # tie
    assert rkv.choose_tail_mode(0, 1.0, 100.0) == rkv.RKV_TAIL_LIFT       # nothing to move
    rng = np.random.default_rng(7)
    for _ in range(200):
        b, h, c = int(rng.integers(1, 1 << 40)), float(rng.uniform(0.1, 200)), float(rng.uniform(0.1, 200))
        want = rkv.RKV_TAIL_HOST if b / c < b / h else rkv.RKV_TAIL_LIFT
        assert rkv.choose_tail_mode(b, h, c) == want
    for bad in ((-1, 1.0, 1.0), (1, 0.0, 1.0), (1, 1.0, -2.0), (1, float("inf"), 1.0), (1, 1.0, float("nan"))):
        with pytest.raises(_lib.RkvError) as e:
            rkv.choose_tail_mode(*bad)
        assert e.value.status == _lib.RKV_ERR_ARG


@pytest.mark.parametrize("dk,dv", [(64, 64), (256, 256), (512, 512), (576, 512)])
@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_F16, gen.TYPE_F16)])
def test_other_head_dims(rkv, dk, dv, kt, vt):
    """Head dims other than 128 (patch 0070: the streaming op's shapes): 10 query heads on 2 KV
    heads, 2 queries, a causal limit and a mask, cell- and head-major."""
    rng = np.random.default_rng(dk + 7 * kt)
    n_q, n_cells, kv_pos0 = 2, 1500, 300
    q, k, v = gen.draw_qkv(rng, 10, n_q, 2, n_cells, d=dk, dv=dv, k_type=kt, v_type=vt)
    mask = gen.random_mask_f16(rng, n_q, kv_pos0 + n_cells, p_hidden=0.2)
    scale = 1 / np.sqrt(dk)
    q_pos0 = kv_pos0 + n_cells - 400  # the last 400 cells are after query 0's position
    causal = oracle.causal_mask(n_q, kv_pos0 + n_cells, q_pos0)[:, kv_pos0:]
    ref = oracle_partial(q, k, v, kt, vt, mask[:, kv_pos0:].astype(np.float64) + causal, scale=scale)
    for layout in ("cell", "head"):
        host = run_host(rkv, q, k, v, kt, vt, mask=mask, kv_pos0=kv_pos0, q_pos0=q_pos0, scale=scale,
                        layout=layout)
        check_partial(host, ref, f"d={dk}/{dv} {layout}")

