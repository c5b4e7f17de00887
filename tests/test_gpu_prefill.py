"""GPU parity of rkv_attn_prefill (MFMA segment kernel) against the fp64 oracle: causal chunks
at the end of the cache, window + lifted tail tiles, masks, ragged query/key counts, quant
types, outlier keys, and the full-size 512-query chunk checked on sampled rows."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    return Runner()


def chunk(num=5, n_kv=1664, n_q=160, wc=1024, tile=512, **over):
    """Prefill-chunk workload at an oracle-sized length: the chunk's n_q queries are the last
    n_q positions of the cache (q_pos0 = n_kv - n_q)."""
    base = gen.WORKLOADS[num]
    sd = max(1, base["n_kv"] // n_kv)
    w = gen.make_workload(num, scale_down=sd, n_q=n_q, **over)
    w["wc"], w["tile_kv"] = min(wc, w["n_kv"]), tile
    w["q_pos0"] = w["n_kv"] - n_q
    return w


def causal_ref(w, q_pos0=None, mask=None):
    q_pos0 = w["q_pos0"] if q_pos0 is None else q_pos0
    n_q = w["q"].shape[1]
    m = oracle.causal_mask(n_q, w["n_kv"], q_pos0) if q_pos0 >= 0 else np.zeros((n_q, w["n_kv"]))
    if mask is not None:
        m = m + np.asarray(mask, dtype=np.float64)
    return oracle_decode(w, mask=m)


def test_q8q4_causal_chunk_window_and_tail_tiles(run):
    # 40/8 heads, 160 queries (800 rows per KV head: 6 full row tiles + a ragged one),
    # window 1024 + host tail 640 in tiles 512 + 128 (causal triangle in the last tile)
    w = chunk()
    step(f"prefill q8q4 n_q=160 n_kv={w['n_kv']} wc=1024 tile=512 host tail, causal")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="q8q4 causal")
    st = run.ctx.stats()
    assert st["kernel_variant"] == 1 and st["n_tail_tiles"] == 2


@pytest.mark.parametrize("tail", ["device", "host"])
def test_f16_chunk_config1_heads(run, tail):
    w = chunk(num=1, n_kv=4096, n_q=64, wc=2048, tile=1024)
    step(f"prefill f16 8/2 heads n_q=64 n_kv=4096 tail={tail}")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail=tail)
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what=f"f16 {tail}")


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_F16), (gen.TYPE_F16, gen.TYPE_Q4_0),
                                   (gen.TYPE_F16, gen.TYPE_F16)])
def test_type_combinations(run, kt, vt):
    w = chunk(n_kv=1664, n_q=48, wc=900, tile=333, k_type=kt, v_type=vt)
    step(f"prefill k={kt} v={vt} n_q=48 wc=900 tile=333")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="types")


@pytest.mark.parametrize("tile", [31, 64, 100, 4096])
def test_tile_sweep_ragged(run, tile):
    w = chunk(n_kv=1664, n_q=40, wc=1333, tile=tile)
    step(f"prefill q8q4 wc=1333 tile={tile}")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what=f"tile {tile}")


def test_no_causal_with_mask_and_empty_rows(run):
    w = chunk(n_kv=1664, n_q=24, wc=1000, tile=400)
    rng = np.random.default_rng(11)
    mask = gen.random_mask_f16(rng, 24, w["n_kv"], p_hidden=0.35)
    mask[5, :] = -np.inf  # query 5 sees nothing
    mask[17, 1000:] = -np.inf  # query 17 sees the window only
    step("prefill q8q4 mask only (q_pos0=-1), empty row")
    O, L = run.decode(w, prefill=True, q_pos0=-1, tail="host", mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="mask")
    assert np.all(O[5] == 0) and np.all(L[5] == -np.inf)


def test_causal_plus_mask(run):
    w = chunk(n_kv=1664, n_q=40, wc=1024, tile=512)
    rng = np.random.default_rng(12)
    mask = gen.random_mask_f16(rng, 40, w["n_kv"], p_hidden=0.2)
    step("prefill q8q4 causal + mask")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host", mask=mask)
    Oref, Lref = causal_ref(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="causal+mask")


def test_chunk_in_the_middle_sees_no_later_keys(run):
    """q_pos0 inside the window: whole tail tiles lie after every query and contribute nothing."""
    w = chunk(n_kv=1664, n_q=64, wc=1024, tile=256)
    step("prefill q8q4 q_pos0=500 (tail invisible)")
    O, L = run.decode(w, prefill=True, q_pos0=500, tail="host")
    Oref, Lref = causal_ref(w, q_pos0=500)
    assert_close(O, L, Oref, Lref, what="middle")


@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(8, 8, 9), (8, 2, 3), (6, 2, 50), (7, 1, 40), (40, 8, 2)])
def test_group_shapes(run, n_head, n_head_kv, n_q):
    w = chunk(n_kv=1664, n_q=n_q, wc=1200, tile=300, n_head=n_head, n_head_kv=n_head_kv)
    step(f"prefill gqa shape {n_head}/{n_head_kv} n_q={n_q}")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="gqa")


def test_outlier_keys_exact_k(run):
    """Every 17th key scaled x30: q8_0 K enters the MFMA as two binary16 parts, so its large
    values are not rounded."""
    rng = gen.rng_for(98)
    n_q, n_kv = 64, 1600
    q, k, v = gen.draw_qkv(rng, 40, n_q, 8, n_kv, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0, outlier_every=17)
    w = dict(n_head=40, n_head_kv=8, q=q, k=k, v=v, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0,
             scale=1 / np.sqrt(128), n_kv=n_kv, wc=1000, tile_kv=300, q_pos0=n_kv - n_q)
    step("prefill outlier keys x30 every 17th")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="outliers")


def test_head_major_layout(run):
    w = chunk(n_kv=1664, n_q=32, wc=1024, tile=512)
    step("prefill q8q4 head-major layout, device tail")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="device", layout="head")
    Oref, Lref = causal_ref(w)
    assert_close(O, L, Oref, Lref, what="head-major")


def test_partial_entry_uses_mfma_kernel(run):
    import torch
    import tiered_kv_cache_split_amd as rkv
    w = chunk(n_kv=1664, n_q=32, wc=1664, tile=512)
    seg = slice(200, 1500)
    q_pos0 = 1400
    step("attn_partial prefill-sized (mfma) kv_pos0=200 q_pos0=1400")
    qd = dev(w["q"])
    kd, vd = dev(w["k"][seg]), dev(w["v"][seg])
    part = torch.empty((32 * w["n_head"], 130), dtype=torch.float32, device="cuda")
    run.ctx.attn_partial(rkv.q_desc(qd), rkv.kv_desc(kd, w["k_type"]), rkv.kv_desc(vd, w["v_type"]), None, 200,
                         q_pos0, w["scale"], part)
    torch.cuda.synchronize()
    assert run.ctx.stats()["kernel_variant"] == 1
    P = part.cpu().numpy().astype(np.float64)
    qv = oracle.q_values(w["q"])
    kv = oracle.kv_values(w["k_type"], w["k"][seg])
    vv = oracle.kv_values(w["v_type"], w["v"][seg])
    m = oracle.causal_mask(32, 1500, q_pos0)[:, 200:1500]
    M, S, VKQ = oracle.partial(qv, kv, vv, w["scale"], m)
    # compare as (O = VKQ/S, LSE = M + ln S), the quantities the tolerances are defined on
    Og, Lg = P[:, 2:] / P[:, 1:2], P[:, 0] + np.log(P[:, 1])
    Or, Lr = (VKQ / S[..., None]).reshape(-1, 128), (M + np.log(S)).reshape(-1)
    assert_close(Og, Lg, Or, Lr, what="partial")


def test_full_size_chunk_all_queries(run):
    """The 512-query chunk against n_kv=106496 (window 65536 + host tail 32768 + 8192), in the
    launch configuration the benchmark times; the oracle checks all 512 queries (in chunks of 64)
    of every query head of KV heads 0 and 5, over all keys."""
    w = gen.make_workload(5)
    step("prefill full size n_q=512 n_kv=106496 wc=65536 tile=32768 host tail")
    O, L = run.decode(w, prefill=True, q_pos0=w["q_pos0"], tail="host")
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    gqa = w["n_head"] // w["n_head_kv"]
    mask = oracle.causal_mask(512, w["n_kv"], w["q_pos0"])
    for g in (0, 5):
        kv = oracle.kv_values(w["k_type"], w["k"][:, g:g + 1])
        vv = oracle.kv_values(w["v_type"], w["v"][:, g:g + 1])
        for i0 in range(0, 512, 64):
            qi = np.arange(i0, i0 + 64)
            qv = oracle.q_values(w["q"][g * gqa:(g + 1) * gqa][:, qi])
            Oref, Lref = oracle.attention(qv, kv, vv, w["scale"], mask[qi])
            assert_close(O[qi][:, g * gqa:(g + 1) * gqa], L[qi][:, g * gqa:(g + 1) * gqa], Oref, Lref,
                         what=f"full size head group {g} queries {i0}..{i0 + 63}")
