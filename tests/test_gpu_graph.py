"""Decode inside a captured HIP graph: after rkv_reserve nothing is allocated in a call, so a
window + lifted-tail decode (copy stream, ring slots, events) and a resident decode can be
captured once and replayed.  Every replay, with eager work and synchronisation between
replays, must equal the eager call bit for bit (same kernels, same split) and the oracle to
the spec tolerances.  Growth needed during capture, and the host tail mode, report
RKV_ERR_CAPTURE instead of allocating."""
import numpy as np
import pytest

import rkv_inputs as gen
from rkv_testutil import assert_close, dev, oracle_decode, pinned, step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def tensors(rkv, w, tail):
    wc = w["wc"]
    t = {"q": dev(w["q"]), "kw": dev(w["k"][:wc]), "vw": dev(w["v"][:wc])}
    if tail:
        t["kt"], t["vt"] = pinned(w["k"][wc:]), pinned(w["v"][wc:])
    n_q, n_head = w["q"].shape[1], w["n_head"]
    t["o"] = torch.zeros((n_q, n_head, 128), dtype=torch.float32, device="cuda")
    t["lse"] = torch.zeros((n_q, n_head), dtype=torch.float32, device="cuda")
    d = {"q": rkv.q_desc(t["q"]), "kw": rkv.kv_desc(t["kw"], w["k_type"]), "vw": rkv.kv_desc(t["vw"], w["v_type"]),
         "kt": rkv.kv_desc(t["kt"], w["k_type"]) if tail else None,
         "vt": rkv.kv_desc(t["vt"], w["v_type"]) if tail else None}
    return t, d


def decode(ctx, w, t, d, stream=None):
    ctx.attn_decode(d["q"], d["kw"], d["vw"], d["kt"], d["vt"], None, w["wc"], w["tile_kv"], w["scale"], t["o"],
                    t["lse"], stream=stream)


def reserve_for(ctx, w):
    tile = min(w["tile_kv"], w["n_kv"] - w["wc"]) if w["n_kv"] > w["wc"] else 1
    kb = tile * w["n_head_kv"] * gen.row_bytes(w["k_type"], 128)
    vb = tile * w["n_head_kv"] * gen.row_bytes(w["v_type"], 128)
    ctx.reserve(kb, vb, 2, 2048 * w["n_head"] * w["q"].shape[1] * 130)


@pytest.mark.parametrize("num,sd,tail,in_place", [(3, 32, True, False), (1, 1, True, False), (2, 16, False, False),
                                                  (1, 1, True, True)])
def test_decode_graph_replays(num, sd, tail, in_place):
    """in_place: the 2 MB tail read in place by the segment kernels (the automatic mode's choice
    for a small decode tail); otherwise lifted through the ring."""
    import tiered_kv_cache_split_amd as rkv
    w = gen.make_workload(num, scale_down=sd)
    if not tail:
        w["wc"] = w["n_kv"]
    ctx = rkv.Context(0)
    ctx.set_direct_tail_max(8 << 20 if in_place else 0)
    try:
        reserve_for(ctx, w)
        t, d = tensors(rkv, w, tail)
        step(f"graph: eager decode workload {num}/{sd} tail={tail}")
        decode(ctx, w, t, d)
        torch.cuda.synchronize()
        if tail:
            assert (ctx.stats()["lift_mode"] == rkv.RKV_LIFT_DIRECT) == in_place
        O0, L0 = t["o"].cpu().numpy().copy(), t["lse"].cpu().numpy().copy()
        Oref, Lref = oracle_decode(w)
        assert_close(O0, L0, Oref, Lref, what="eager")
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        step(f"graph: capture workload {num}/{sd}")
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                decode(ctx, w, t, d, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda")
        for r in range(4):
            t["o"].fill_(float("nan"))
            t["lse"].fill_(float("nan"))
            junk.mul_(1.0001).add_(0.5)  # eager work between replays
            torch.cuda.synchronize()
            step(f"graph: replay {r}")
            g.replay()
            torch.cuda.synchronize()
            O, L = t["o"].cpu().numpy(), t["lse"].cpu().numpy()
            assert np.array_equal(O, O0) and np.array_equal(L, L0), f"replay {r} differs from the eager call"
        del g
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_growth_inside_capture_is_refused():
    """A fresh context has no ring or workspace: capturing a lifted-tail decode must fail with
    RKV_ERR_CAPTURE before any allocation, and the context works eagerly afterwards."""
    import tiered_kv_cache_split_amd as rkv
    from tiered_kv_cache_split_amd import _lib
    w = gen.make_workload(1)
    ctx = rkv.Context(0)
    ctx.set_direct_tail_max(0)  # the tails below are lifted (the small ones would be read in place)
    try:
        t, d = tensors(rkv, w, True)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        step("graph: capture without reserve")
        err = None
        with torch.cuda.stream(side):
            g.capture_begin()
            try:
                decode(ctx, w, t, d, stream=side)
            except _lib.RkvError as e:
                err = e
            finally:
                g.capture_end()
        torch.cuda.synchronize()
        assert err is not None and err.status == _lib.RKV_ERR_CAPTURE, err
        step("graph: eager decode after the refused capture")
        decode(ctx, w, t, d)
        torch.cuda.synchronize()
        Oref, Lref = oracle_decode(w)
        assert_close(t["o"].cpu().numpy(), t["lse"].cpu().numpy(), Oref, Lref, what="after refused capture")
        # the host tail partial needs the host mid-call: refused inside capture as well
        reserve_for(ctx, w)
        ctx.set_tail_mode(rkv.RKV_TAIL_HOST, 4)
        g2 = torch.cuda.CUDAGraph()
        err = None
        step("graph: capture with the host tail mode")
        with torch.cuda.stream(side):
            g2.capture_begin()
            try:
                decode(ctx, w, t, d, stream=side)
            except _lib.RkvError as e:
                err = e
            finally:
                g2.capture_end()
        torch.cuda.synchronize()
        assert err is not None and err.status == _lib.RKV_ERR_CAPTURE, err
    finally:
        torch.cuda.synchronize()
        ctx.close()


@pytest.mark.parametrize("kt,vt", [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0)])
def test_rows_graph_replays_with_new_lists(kt, vt):
    """A captured rkv_attn_rows replayed after the lists in its buffer changed (longer, shorter,
    all padding): every replay rescans the lists' extents and must match the oracle for its own
    lists."""
    import tiered_kv_cache_split_amd as rkv
    from rkv_testutil import oracle_rows
    rng = gen.rng_for(91)
    n_pool, n_kv = 2500, 2000
    q = gen.draw_normal(rng, (2, 32, 1, 128)).astype(np.float16)
    k = gen.pack(kt, gen.draw_normal(rng, (n_pool, 8, 128)))
    v = gen.pack(vt, gen.draw_normal(rng, (n_pool, 8, 128)))
    ctx = rkv.Context(0)
    try:
        ctx.reserve(0, 0, 0, 1024 * 2 * 32 * 130)
        qd, kd, vd = dev(q), dev(k), dev(v)
        kvr = dev(gen.rows_lists(rng, n_pool, (1500, 1900), n_kv, shuffle=True))
        o = torch.empty((2, 1, 32, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((2, 1, 32), dtype=torch.float32, device="cuda")

        def call(stream=None):
            ctx.attn_rows(rkv.q_desc(qd), rkv.kv_desc(kd, kt), rkv.kv_desc(vd, vt), kvr, n_kv, None,
                          1 / np.sqrt(128), o, lse, stream=stream)

        step(f"graph rows {kt}/{vt}: eager call, then capture")
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                call(stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for lengths in ((2000, 300), (100, 1700), (0, 0), (1999, 2000)):
            rows = gen.rows_lists(rng, n_pool, lengths, n_kv, shuffle=True)
            kvr.copy_(torch.from_numpy(rows))
            o.fill_(float("nan"))
            torch.cuda.synchronize()
            step(f"graph rows {kt}/{vt}: replay with lists {lengths}")
            g.replay()
            torch.cuda.synchronize()
            w = dict(q=q, k=k, v=v, kv_rows=rows, mask=None, k_type=kt, v_type=vt, scale=1 / np.sqrt(128))
            Oref, Lref = oracle_rows(w, mask=None)
            assert_close(o.cpu().numpy(), lse.cpu().numpy(), Oref, Lref, what=f"graph rows {lengths}")
        del g
    finally:
        torch.cuda.synchronize()
        ctx.close()
