"""GPU parity of rkv_attn_decode / rkv_lse_merge / rkv_attn_partial against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import LSE_TOL, O_TOL, Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    return Runner()


def small(num, n_kv, wc, tile, **over):
    """Workload `num` at an oracle-sized length (several chunks, ragged ends)."""
    w = gen.make_workload(num, **over)
    if w["n_kv"] != n_kv:
        base = gen.WORKLOADS[num]
        sd = max(1, base["n_kv"] // n_kv)
        w = gen.make_workload(num, scale_down=sd, **over)
    w["wc"], w["tile_kv"] = min(wc, w["n_kv"]), tile
    return w


def test_f16_window_only_config1_shape(run):
    w = gen.make_workload(1)
    step("decode f16 n_kv=4096 window only")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="window only")


@pytest.mark.parametrize("tail", ["device", "host"])
def test_f16_window_plus_tail_config1(run, tail):
    w = gen.make_workload(1)
    step(f"decode f16 config1 wc=2048 tail={tail} tile=1024")
    O, L = run.decode(w, tail=tail)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"tail {tail}")
    st = run.ctx.stats()
    if tail == "host":
        assert st["n_tail_tiles"] == 2 and st["lift_bytes"] == 2048 * 2 * 2 * 256


@pytest.mark.parametrize("tile", [31, 256, 512, 768, 1024, 32768])
def test_tile_sweep_wc_not_multiple_of_256(run, tile):
    w = gen.make_workload(1)
    step(f"decode f16 wc=1333 tile={tile}")
    O, L = run.decode(w, wc=1333, tile_kv=tile, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"tile {tile}")


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
                                   (gen.TYPE_F16, gen.TYPE_Q4_0)])
def test_quant_decode_ragged(run, kt, vt):
    w = gen.make_workload(2, scale_down=32, k_type=kt, v_type=vt)  # n_kv 4096
    step(f"decode k={kt} v={vt} n_kv=4096 wc=2333 tile=700")
    O, L = run.decode(w, wc=2333, tile_kv=700, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="quant")


@pytest.mark.parametrize("layout", ["cell", "head"])
def test_quant_layouts_and_device_tail(run, layout):
    w = gen.make_workload(3, scale_down=64)  # n_kv 4096, wc 2048, tile 512
    step(f"decode q8q4 layout={layout} device tail")
    O, L = run.decode(w, tail="device", layout=layout)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=layout)
    step(f"decode q8q4 layout={layout} host tail")
    O2, L2 = run.decode(w, tail="host", layout=layout)
    assert_close(O2, L2, Oref, Lref, what=layout + " host")


@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(8, 8, 1), (8, 4, 1), (16, 2, 1), (8, 2, 2), (6, 2, 1),
                                                  (7, 1, 1)])
def test_group_shapes(run, n_head, n_head_kv, n_q):
    w = gen.make_workload(1, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)
    step(f"decode gqa shape {n_head}/{n_head_kv} n_q={n_q}")
    O, L = run.decode(w, wc=1500, tile_kv=1000, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="gqa")


def test_mask_with_hidden_keys_and_empty_row(run):
    w = gen.make_workload(1, n_q=2, n_head=8, n_head_kv=2)
    rng = np.random.default_rng(3)
    mask = gen.random_mask_f16(rng, 2, w["n_kv"], p_hidden=0.4)
    mask[1, :] = -np.inf  # query 1 sees nothing
    step("decode masked, one empty row")
    O, L = run.decode(w, wc=2048, tile_kv=1024, tail="host", mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="mask")
    assert np.all(O[1] == 0) and np.all(L[1] == -np.inf)


def test_mask_sliced_at_global_position(run):
    """Hiding exactly the tail columns must give the window-only result (mask column = global key)."""
    w = gen.make_workload(1)
    mask = np.zeros((1, w["n_kv"]), np.float16)
    mask[0, 2048:] = -np.inf
    step("decode mask hides tail")
    O, L = run.decode(w, wc=2048, tile_kv=512, tail="host", mask=mask)
    w2 = dict(w)
    w2["k"], w2["v"], w2["n_kv"] = w["k"][:2048], w["v"][:2048], 2048
    Oref, Lref = oracle_decode(w2)
    assert_close(O, L, Oref, Lref, what="global mask")


def test_outlier_keys(run):
    rng = gen.rng_for(99)
    q, k, v = gen.draw_qkv(rng, 8, 1, 2, 3000, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0, outlier_every=17)
    w = dict(n_head=8, n_head_kv=2, q=q, k=k, v=v, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0,
             scale=1 / np.sqrt(128), n_kv=3000, wc=1800, tile_kv=600)
    step("decode outlier keys x30 every 17th")
    O, L = run.decode(w, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="outliers")


def test_empty_tail_equals_single_resident(run):
    w = gen.make_workload(1)
    step("decode empty tail vs window only")
    O1, L1 = run.decode(w, wc=4096, tail=None)
    w2 = dict(w)
    O2, L2 = run.decode(w2, wc=4096, tail="host")  # zero-length tail slice
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("num,sd,layout", [(1, 1, "cell"), (3, 64, "cell"), (3, 64, "head"), (3, 32, "cell")])
def test_kernel_lift(run, num, sd, layout):
    """Tail tiles lifted by the copy kernel (RKV_LIFT_KERNEL) instead of the DMA engine."""
    w = gen.make_workload(num, scale_down=sd)
    run.ctx.set_lift_mode(run.rkv.RKV_LIFT_KERNEL)
    try:
        step(f"decode kernel lift workload {num}/{sd} layout {layout} wc {w['wc']} tile {w['tile_kv']}")
        O, L = run.decode(w, tail="host", layout=layout)
        st = run.ctx.stats()
    finally:
        run.ctx.set_lift_mode(run.rkv.RKV_LIFT_AUTO)
    assert st["lift_mode"] == 2 and st["n_tail_tiles"] >= 2
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"kernel lift {num}/{sd} {layout}")


def test_automatic_lift_mode_per_entry_point(run):
    """Default lift: decode tails through the copy kernel, prefill tails through the DMA engine."""
    w = gen.make_workload(3, scale_down=64)
    step("automatic lift mode: decode")
    O, L = run.decode(w, tail="host")
    assert run.ctx.stats()["lift_mode"] == run.rkv.RKV_LIFT_KERNEL
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="automatic lift, decode")
    w5 = gen.make_workload(5, scale_down=52)
    step("automatic lift mode: prefill")
    O, L = run.decode(w5, tail="host", prefill=True, q_pos0=w5["q_pos0"])
    assert run.ctx.stats()["lift_mode"] == run.rkv.RKV_LIFT_BULK
    Oref, Lref = oracle_decode(w5, mask=oracle.causal_mask(w5["n_q"], w5["n_kv"], w5["q_pos0"]))
    assert_close(O, L, Oref, Lref, what="automatic lift, prefill")


def test_back_to_back_calls_reuse_slots(run):
    """Several calls with 4 tail tiles through a 2-slot ring, queued without syncing between them,
    each against other work on the stream (the reused-slot race classes)."""
    import torch
    ws = [gen.make_workload(3, scale_down=64) for _ in range(1)]
    w = ws[0]
    Oref, Lref = oracle_decode(w)
    keep = []
    outs = []
    step("decode back-to-back 5 calls, 4 tiles, 2 slots")
    rkv = run.rkv
    q = dev(w["q"])
    kw, vw = dev(w["k"][:2048]), dev(w["v"][:2048])
    from rkv_testutil import pinned
    kt, vt = pinned(w["k"][2048:]), pinned(w["v"][2048:])
    junk = torch.randn(4096, 4096, device="cuda")
    for it in range(5):
        o = torch.empty((1, w["n_head"], 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, w["n_head"]), dtype=torch.float32, device="cuda")
        junk = junk @ junk.T * 1e-3  # unrelated compute on the same stream
        run.ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kw, w["k_type"]), rkv.kv_desc(vw, w["v_type"]),
                            rkv.kv_desc(kt, w["k_type"]), rkv.kv_desc(vt, w["v_type"]), None, 2048, 512,
                            w["scale"], o, lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for o, lse in outs:
        assert_close(o.cpu().numpy(), lse.cpu().numpy(), Oref, Lref, what="back-to-back")


def test_lse_merge_of_oracle_partials(run):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, 3, 128))
    k = rng.standard_normal((2, 900, 128))
    v = rng.standard_normal((2, 900, 128))
    bounds = [0, 100, 100, 555, 900]
    parts = [oracle.partial(q, k[:, a:b], v[:, a:b], 0.09, None) for a, b in zip(bounds[:-1], bounds[1:])]
    n_rows = 3 * 8
    P = np.zeros((len(parts), n_rows, 130), np.float32)
    for s, (M, S, VKQ) in enumerate(parts):
        P[s, :, 0] = M.reshape(-1)
        P[s, :, 1] = S.reshape(-1)
        P[s, :, 2:] = VKQ.reshape(n_rows, 128)
    import torch
    import tiered_kv_cache_split_amd as rkv
    Pd = dev(P)
    o = torch.empty((n_rows, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_rows,), dtype=torch.float32, device="cuda")
    step("lse merge of oracle partials")
    rkv.lse_merge(Pd, len(parts), n_rows, o, lse)
    torch.cuda.synchronize()
    Oref, Lref = oracle.merge(parts)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), Oref.reshape(n_rows, 128), Lref.reshape(-1), what="merge")


@pytest.mark.parametrize("n_seg,n_rows", [(17, 24), (100, 40), (256, 40), (257, 24), (600, 8), (256, 1100)])
def test_lse_merge_many_segments(run, n_seg, n_rows):
    """The merge kernels for many segments (one thread per segment and head_dim part, and the
    tiled one past 256 segments) against the oracle merge, with empty segments (M = -inf,
    S = 0) scattered in and one row whose segments are all empty."""
    import torch
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(1000 + n_seg)
    M = rng.uniform(-6.0, 6.0, (n_seg, n_rows))
    S = rng.uniform(0.5, 40.0, (n_seg, n_rows))
    VKQ = rng.standard_normal((n_seg, n_rows, 128)) * S[..., None]
    empty = rng.random((n_seg, n_rows)) < 0.2
    empty[:, 3] = True
    M[empty] = -np.inf
    S[empty] = 0.0
    VKQ[empty] = 0.0
    P = np.zeros((n_seg, n_rows, 130), np.float32)
    P[:, :, 0], P[:, :, 1], P[:, :, 2:] = M, S, VKQ
    parts = [(P[s, :, 0].astype(np.float64)[None], P[s, :, 1].astype(np.float64)[None],
              P[s, :, 2:].astype(np.float64)[None]) for s in range(n_seg)]
    Oref, Lref = oracle.merge(parts)
    o = torch.empty((n_rows, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_rows,), dtype=torch.float32, device="cuda")
    step(f"lse merge of {n_seg} synthetic partials x {n_rows} rows")
    rkv.lse_merge(dev(P), n_seg, n_rows, o, lse)
    torch.cuda.synchronize()
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), Oref.reshape(n_rows, 128), Lref.reshape(-1), what="merge")


def test_attn_partial_matches_oracle_partial(run):
    import torch
    import tiered_kv_cache_split_amd as rkv
    w = gen.make_workload(2, scale_down=64)  # 2048 cells q8q4
    step("attn_partial q8q4 segment at kv_pos0=5000")
    seg = slice(300, 1700)
    mask = gen.random_mask_f16(np.random.default_rng(8), 1, 5000 + 1400, p_hidden=0.2)
    q = dev(w["q"])
    kd, vd = dev(w["k"][seg]), dev(w["v"][seg])
    md = dev(mask)
    part = torch.empty((w["n_head"], 130), dtype=torch.float32, device="cuda")
    run.ctx.attn_partial(rkv.q_desc(q), rkv.kv_desc(kd, w["k_type"]), rkv.kv_desc(vd, w["v_type"]),
                         rkv.mask_desc(md), 5000, -1, w["scale"], part)
    torch.cuda.synchronize()
    P = part.cpu().numpy().astype(np.float64)
    qv = oracle.q_values(w["q"])
    kv = oracle.kv_values(w["k_type"], w["k"][seg])
    vv = oracle.kv_values(w["v_type"], w["v"][seg])
    M, S, VKQ = oracle.partial(qv, kv, vv, w["scale"], mask[:, 5000:].astype(np.float64))
    # compare the normalised forms (a partial is defined up to the common factor e^M)
    assert np.allclose(P[:, 0] + np.log(P[:, 1]), (M + np.log(S))[0], atol=LSE_TOL)
    assert np.abs(P[:, 2:] / P[:, 1:2] - (VKQ / S[..., None])[0]).max() <= O_TOL


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_F16, gen.TYPE_F16)])
def test_large_logits_need_the_true_running_max(run, kt, vt):
    """Unscaled outlier scores (hundreds): exp overflows unless every chunk's wave max is the
    true maximum, so a wrong cross-lane reduction shows up as inf/NaN or a large error."""
    rng = gen.rng_for(98)
    q, k, v = gen.draw_qkv(rng, 8, 1, 2, 2500, k_type=kt, v_type=vt, outlier_every=17, outlier_scale=30.0)
    w = dict(n_head=8, n_head_kv=2, q=q, k=k, v=v, k_type=kt, v_type=vt, scale=1.0, n_kv=2500, wc=1700,
             tile_kv=500)
    step(f"decode large logits k={kt} v={vt}")
    O, L = run.decode(w, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="large logits")


# ---- matrix-core decode kernel (cell-major q8_0 K / q4_0 V, eight KV heads per workgroup)

@pytest.mark.parametrize("n_head_kv,n_head,n_q", [(4, 4, 1), (4, 20, 1), (4, 32, 1), (4, 8, 3), (2, 2, 1),
                                                  (2, 10, 1), (2, 16, 1), (6, 24, 1), (12, 96, 1)])
def test_mma_decode_smaller_head_groups(run, n_head_kv, n_head, n_q):
    """Groups of 4 or 2 KV heads per workgroup (n_head_kv not a multiple of 8)."""
    w = gen.make_workload(2, scale_down=32, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q)
    step(f"decode q8q4 {n_head_kv} kv heads n_head={n_head} n_q={n_q} wc=2500 tile=900")
    O, L = run.decode(w, wc=2500, tile_kv=900, tail="host")
    assert run.ctx.stats()["kernel_variant"] == 3
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"mma kv heads {n_head_kv}")


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16)])
@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(24, 4, 1), (28, 4, 1), (32, 4, 1), (8, 1, 1), (4, 1, 2)])
def test_many_rows_per_head_major_kv_head(run, kt, vt, n_head, n_head_kv, n_q):
    """Head-major caches with q8_0 K and 6 to 8 rows per KV head run on the head-dim kernel at
    128 (rows in groups of 8)."""
    w = gen.make_workload(2, scale_down=32, n_head=n_head, n_head_kv=n_head_kv, n_q=n_q, k_type=kt, v_type=vt)
    mask = gen.random_mask_f16(np.random.default_rng(n_head + n_q), n_q, w["n_kv"], p_hidden=0.2)
    step(f"decode head-major k={kt} v={vt} heads {n_head}/{n_head_kv} n_q {n_q}")
    O, L = run.decode(w, wc=2500, tile_kv=900, tail="host", layout="head", mask=mask)
    assert run.ctx.stats()["kernel_variant"] == 5
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    assert_close(O, L, Oref, Lref, what=f"head-major {n_head}/{n_head_kv}/{n_q}")

@pytest.mark.parametrize("n_head,n_q", [(8, 1), (16, 1), (24, 1), (32, 1), (40, 1), (48, 1), (56, 1), (64, 1),
                                        (32, 2), (16, 3)])
def test_mma_decode_row_counts(run, n_head, n_q):
    w = gen.make_workload(2, scale_down=32, n_head=n_head, n_q=n_q)  # n_kv 4096, 8 KV heads
    step(f"decode q8q4 8 kv heads n_head={n_head} n_q={n_q} wc=2500 tile=900")
    O, L = run.decode(w, wc=2500, tile_kv=900, tail="host")
    assert run.ctx.stats()["kernel_variant"] == 3  # every row count here is at most 8 per KV head
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"mma rows {n_head}x{n_q}")


def test_mma_decode_mask_empty_row_ragged(run):
    w = gen.make_workload(2, scale_down=32, n_q=1)
    w = dict(w)
    n_kv = 3001
    w["k"], w["v"], w["n_kv"] = w["k"][:n_kv], w["v"][:n_kv], n_kv
    rng = np.random.default_rng(21)
    mask = gen.random_mask_f16(rng, 1, n_kv, p_hidden=0.3)
    step("decode q8q4 8 kv heads, mask, n_kv=3001 window only")
    O, L = run.decode(w, wc=n_kv, tail=None, mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what="mma mask")
    mask2 = np.full((1, n_kv), -np.inf, np.float16)
    step("decode q8q4 8 kv heads, everything masked")
    O2, L2 = run.decode(w, wc=n_kv, tail=None, mask=mask2)
    assert np.all(O2 == 0) and np.all(L2 == -np.inf)


def test_mma_decode_outlier_keys(run):
    rng = gen.rng_for(97)
    q, k, v = gen.draw_qkv(rng, 40, 1, 8, 3000, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0, outlier_every=17)
    w = dict(n_head=40, n_head_kv=8, q=q, k=k, v=v, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0,
             scale=1 / np.sqrt(128), n_kv=3000, wc=1800, tile_kv=600)
    step("decode q8q4 8 kv heads outlier keys")
    O, L = run.decode(w, tail="host")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="mma outliers")


def test_mma_decode_two_head_groups(run):
    w = gen.make_workload(2, scale_down=32, n_head=32, n_head_kv=16)
    step("decode q8q4 16 kv heads (two groups of 8)")
    O, L = run.decode(w, wc=3000, tile_kv=1096, tail="device")
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what="mma head groups")


def test_full_size_config2_all_heads(run):
    """n_kv = 131072 fully resident, 40/8 heads q8_0/q4_0, in the benchmark's launch configuration;
    the oracle checks every query head over all keys."""
    w = gen.make_workload(2)
    step("decode full size config 2")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    assert run.ctx.stats()["kernel_variant"] == 3  # the matrix-core cell-major kernel
    gqa = w["n_head"] // w["n_head_kv"]
    for g, (Oref, Lref) in oracle_decode(w, heads=list(range(w["n_head_kv"]))).items():
        assert_close(O[:, g * gqa:(g + 1) * gqa], L[:, g * gqa:(g + 1) * gqa], Oref, Lref, what=f"config 2 head {g}")


def test_full_size_config3_all_heads(run):
    """Window 131072 + pinned tail 131072 in 32768-cell tiles (four lifts through the 2-slot ring);
    every query head against the oracle over all 262144 keys."""
    w = gen.make_workload(3)
    step("decode full size config 3")
    O, L = run.decode(w, tail="host")
    st = run.ctx.stats()
    assert st["n_tail_tiles"] == 4 and st["lift_bytes"] == 131072 * 8 * (136 + 72)
    gqa = w["n_head"] // w["n_head_kv"]
    for g, (Oref, Lref) in oracle_decode(w, heads=list(range(w["n_head_kv"]))).items():
        assert_close(O[:, g * gqa:(g + 1) * gqa], L[:, g * gqa:(g + 1) * gqa], Oref, Lref, what=f"config 3 head {g}")


# ---- binary16 matrix-core decode kernel (eight cell-major KV heads per workgroup)

@pytest.mark.parametrize("tail", ["device", "host"])
def test_f16_matrix_core_window_and_tail(run, tail):
    w = gen.make_workload(1, n_head=32, n_head_kv=8)  # n_kv 4096, window 2048, tiles 1024
    rng = np.random.default_rng(31)
    mask = gen.random_mask_f16(rng, 1, w["n_kv"], p_hidden=0.2)
    step(f"decode f16 32/8 heads window 2048 + {tail} tail, mask")
    O, L = run.decode(w, wc=2000, tile_kv=700, tail=tail, mask=mask)
    assert run.ctx.stats()["kernel_variant"] == 4
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"f16 mfma {tail}")


def test_f16_matrix_core_partial_causal(run):
    """attn_partial with the causal rule and gqa 4 x n_q 2 = 8 rows per KV head."""
    import torch
    import tiered_kv_cache_split_amd as rkv
    w = gen.make_workload(1, n_head=32, n_head_kv=8, n_q=2)
    seg = slice(100, 3000)
    q_pos0 = 2500
    step("attn_partial f16 32/8 heads n_q=2 kv_pos0=100 q_pos0=2500")
    qd = dev(w["q"])
    kd, vd = dev(w["k"][seg]), dev(w["v"][seg])
    part = torch.empty((2 * w["n_head"], 130), dtype=torch.float32, device="cuda")
    run.ctx.attn_partial(rkv.q_desc(qd), rkv.kv_desc(kd, w["k_type"]), rkv.kv_desc(vd, w["v_type"]), None, 100,
                         q_pos0, w["scale"], part)
    torch.cuda.synchronize()
    assert run.ctx.stats()["kernel_variant"] == 4
    P = part.cpu().numpy().astype(np.float64)
    qv = oracle.q_values(w["q"])
    kv = oracle.kv_values(w["k_type"], w["k"][seg])
    vv = oracle.kv_values(w["v_type"], w["v"][seg])
    m = oracle.causal_mask(2, 3000, q_pos0)[:, 100:3000]
    M, S, VKQ = oracle.partial(qv, kv, vv, w["scale"], m)
    Og, Lg = P[:, 2:] / P[:, 1:2], P[:, 0] + np.log(P[:, 1])
    Or, Lr = (VKQ / S[..., None]).reshape(-1, 128), (M + np.log(S)).reshape(-1)
    assert_close(Og, Lg, Or, Lr, what="f16 mfma partial causal")
