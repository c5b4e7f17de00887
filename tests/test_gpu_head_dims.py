"""Head dims 64 and 256 (dk = dv) through rkv_attn_decode and rkv_lse_merge against the fp64
oracle: the window + tail split with a lifted (both engines) or device-resident tail, every K/V
type pair, masks with an empty row, the soft-cap, grouped-query rows up to eight per KV head,
the empty cache and the tail's partial computed on the host cores."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu

PAIRS = [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
         (gen.TYPE_F16, gen.TYPE_Q4_0)]


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)
    r.ctx.set_softcap(0.0)
    r.ctx.set_tail_mode(r.rkv.RKV_TAIL_LIFT)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("kt,vt", PAIRS)
@pytest.mark.parametrize("lift", [0, 2])
def test_window_plus_lifted_tail(run, d, kt, vt, lift):
    w = gen.make_workload(1, d=d, k_type=kt, v_type=vt)  # 8/2 heads, n_kv 4096
    run.ctx.set_lift_mode(lift)
    step(f"head dim {d}: k={kt} v={vt} wc=1333 tile=700 lift {lift}")
    O, L = run.decode(w, wc=1333, tile_kv=700, tail="host")
    st = run.ctx.stats()
    # q8_0 / q4_0 at 256 over two packed KV heads: the matrix-core kernel; the rest: vector
    mma = d == 256 and (kt, vt) == (gen.TYPE_Q8_0, gen.TYPE_Q4_0)
    assert st["kernel_variant"] == (3 if mma else 5) and st["n_tail_tiles"] == -(-(4096 - 1333) // 700)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"d={d}")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("layout", ["cell", "head"])
def test_device_tail_and_layouts(run, d, layout):
    w = gen.make_workload(3, scale_down=64, d=d)  # q8_0 K, q4_0 V, 40/8 heads, n_kv 4096, wc 2048
    step(f"head dim {d}: q8q4 layout {layout} device tail")
    O, L = run.decode(w, tail="device", layout=layout)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"d={d} {layout}")
    # head-major rows of 68 / 36 bytes (d = 64) do not start on 8-byte words: the copy kernel
    # hands such spans to the DMA engine
    run.ctx.set_lift_mode(run.rkv.RKV_LIFT_KERNEL)
    step(f"head dim {d}: q8q4 layout {layout} lifted tail, copy kernel")
    O, L = run.decode(w, tail="host", layout=layout)
    assert_close(O, L, Oref, Lref, what=f"d={d} {layout} lifted")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(8, 2, 2), (16, 2, 1), (7, 7, 1)])
def test_mask_gqa_and_empty_row(run, d, n_head, n_head_kv, n_q):
    w = gen.make_workload(1, d=d, n_q=n_q, n_head=n_head, n_head_kv=n_head_kv)
    mask = gen.random_mask_f16(np.random.default_rng(d + n_head), n_q, w["n_kv"], p_hidden=0.4)
    mask[n_q - 1, :] = -np.inf  # the last query sees nothing
    step(f"head dim {d}: mask, heads {n_head}/{n_head_kv}, n_q {n_q}")
    O, L = run.decode(w, wc=2000, tile_kv=1024, tail="host", mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"d={d} mask")
    assert np.all(O[n_q - 1] == 0) and np.all(L[n_q - 1] == -np.inf)


@pytest.mark.parametrize("d", [64, 256])
def test_softcap(run, d):
    w = gen.make_workload(2, scale_down=32, d=d)  # q8q4, 40/8 heads, n_kv 4096
    run.ctx.set_softcap(30.0)
    try:
        step(f"head dim {d}: soft-cap 30, window 2500 + lifted tail")
        O, L = run.decode(w, wc=2500, tile_kv=512, tail="host")
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, softcap=30.0)
    assert_close(O, L, Oref, Lref, what=f"d={d} softcap")


@pytest.mark.parametrize("d", [64, 256])
def test_whole_cache_in_the_tail_and_window_only(run, d):
    w = gen.make_workload(1, d=d, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    Oref, Lref = oracle_decode(w)
    step(f"head dim {d}: wc = 0")
    O, L = run.decode(w, wc=0, tile_kv=999, tail="host")
    assert_close(O, L, Oref, Lref, what=f"d={d} wc=0")
    step(f"head dim {d}: window only")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    assert_close(O, L, Oref, Lref, what=f"d={d} window only")


@pytest.mark.parametrize("d", [64, 256])
def test_empty_cache(d):
    import torch
    import tiered_kv_cache_split_amd as rkv
    ctx = rkv.Context(0)
    try:
        q = dev(np.random.default_rng(3).standard_normal((8, 1, d)).astype(np.float16))
        kw = torch.empty((0, 2, 2 * d), dtype=torch.uint8, device="cuda")
        o = torch.full((1, 8, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
        step(f"head dim {d}: n_kv = 0")
        ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kw, gen.TYPE_F16), rkv.kv_desc(kw, gen.TYPE_F16), None, None,
                        None, 0, 64, 0.125, o, lse)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(lse == -float("inf"))
    finally:
        ctx.close()


@pytest.mark.parametrize("dv", [64, 256])
def test_lse_merge(dv):
    """Partials of the oracle's own segments, one of them empty, merged on the device."""
    import torch
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(dv)
    H, G, N = 8, 2, 300
    q = rng.standard_normal((H, 1, dv))
    k = rng.standard_normal((G, N, dv))
    v = rng.standard_normal((G, N, dv))
    bounds = [0, 100, 100, 217, 300]
    parts = [oracle.partial(q, k[:, a:b], v[:, a:b], 0.1) for a, b in zip(bounds, bounds[1:])]
    n_rows = H
    buf = np.zeros((len(parts), n_rows, 2 + dv), dtype=np.float32)
    for s_, (M, S, VKQ) in enumerate(parts):
        buf[s_, :, 0] = M.reshape(-1)
        buf[s_, :, 1] = S.reshape(-1)
        buf[s_, :, 2:] = VKQ.reshape(n_rows, dv)
    o = torch.empty((n_rows, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_rows,), dtype=torch.float32, device="cuda")
    step(f"lse merge dv {dv}")
    rkv.lse_merge(dev(buf), len(parts), n_rows, o, lse, dv=dv)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(q, k, v, 0.1)
    assert_close(o.cpu().numpy()[None], lse.cpu().numpy()[None], Oref.reshape(1, H, dv), Lref.reshape(1, H),
                 what=f"merge dv={dv}")


@pytest.mark.parametrize("dv,n_seg,n_rows", [(64, 512, 40), (256, 1024, 20), (512, 300, 16), (64, 1500, 8),
                                           (128, 700, 40)])
def test_lse_merge_many_segments(dv, n_seg, n_rows):
    """Synthetic partials, a fifth of them empty (M = -inf, S = 0) with NaN where their values
    would be -- a segment with no keys need not write them -- merged on the device: up to 1024
    segments take the part merge with several segments per thread, more the per-row merge."""
    import torch
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(n_seg + dv)
    M = rng.uniform(-6.0, 6.0, (n_seg, n_rows))
    S = rng.uniform(0.5, 40.0, (n_seg, n_rows))
    VKQ = rng.standard_normal((n_seg, n_rows, dv)) * S[..., None]
    empty = rng.random((n_seg, n_rows)) < 0.2
    empty[:, 3] = True  # every segment of row 3 is empty: O = 0, LSE = -inf
    M[empty], S[empty], VKQ[empty] = -np.inf, 0.0, 0.0
    P = np.zeros((n_seg, n_rows, 2 + dv), np.float32)
    P[:, :, 0], P[:, :, 1], P[:, :, 2:] = M, S, VKQ
    P[empty, 2:] = np.nan
    parts = [(P[s_, :, 0].astype(np.float64)[None], P[s_, :, 1].astype(np.float64)[None],
              np.where(empty[s_][:, None], 0.0, P[s_, :, 2:]).astype(np.float64)[None]) for s_ in range(n_seg)]
    Oref, Lref = oracle.merge(parts)
    o = torch.empty((n_rows, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((n_rows,), dtype=torch.float32, device="cuda")
    step(f"lse merge dv {dv}: {n_seg} segments x {n_rows} rows, empty ones with NaN values")
    rkv.lse_merge(dev(P), n_seg, n_rows, o, lse, dv=dv)
    torch.cuda.synchronize()
    O, L = o.cpu().numpy(), lse.cpu().numpy()
    assert np.all(O[3] == 0) and L[3] == -np.inf
    assert_close(O, L, Oref.reshape(n_rows, dv), Lref.reshape(-1), what=f"merge dv={dv} n_seg={n_seg}")


@pytest.mark.parametrize("d", [64, 256])
def test_host_tail_partial(run, d):
    """The tail's partial on the host cores (RKV_TAIL_HOST) at head dims 64 and 256, merged with
    the window's on the GPU."""
    rkv = run.rkv
    w = gen.make_workload(3, scale_down=64, d=d)  # q8q4, 40/8 heads, n_kv 4096, wc 2048
    run.ctx.set_tail_mode(rkv.RKV_TAIL_HOST)
    try:
        step(f"head dim {d}: host tail partial")
        O, L = run.decode(w, tail="host")
        assert run.ctx.stats()["tail_host"] == 1
    finally:
        run.ctx.set_tail_mode(rkv.RKV_TAIL_LIFT)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"d={d} host tail")
