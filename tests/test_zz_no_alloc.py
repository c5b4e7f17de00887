"""The allocation-free decode entry point (rkv_attn_decode_noalloc) against rkv_attn_decode.

Both run the same kernels; while the planned partials fit the library's static device array
the split plan is the same and the outputs are bit-identical.  Two calls in a row (the second
smaller) check that the shared array is reused correctly; a shape whose planned partials exceed
the array runs with fewer splits and is checked against the fp64 oracle."""
import numpy as np
import pytest

import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu


def run_both(w, run, mask=None):
    import torch
    rkv = run.rkv
    n_head, n_q = w["n_head"], w["q"].shape[1]
    q = dev(w["q"])
    k, v = dev(w["k"]), dev(w["v"])
    md = None
    if mask is not None:
        mt = dev(np.asarray(mask, np.float16))
        md = rkv.mask_desc(mt)
    outs = []
    for which in ("ctx", "noalloc"):
        o = torch.full((n_q, n_head, w["dv"]), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((n_q, n_head), float("nan"), dtype=torch.float32, device="cuda")
        kd, vd = rkv.kv_desc(k, w["k_type"]), rkv.kv_desc(v, w["v_type"])
        if which == "ctx":
            run.ctx.attn_decode(rkv.q_desc(q), kd, vd, None, None, md, w["n_kv"], w["n_kv"], w["scale"], o, lse)
        else:
            rkv.attn_decode_noalloc(rkv.q_desc(q), kd, vd, md, w["scale"], o, lse)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    return outs


def test_noalloc_matches_decode_two_calls():
    run = Runner()
    # call 1: the 40/8-head q8_0 / q4_0 cache of 131072 cells (the matrix-core kernel)
    w1 = gen.make_workload(2)
    step("noalloc call 1: q8_0/q4_0 40/8 heads n_kv 131072")
    (O1, L1), (N1, M1) = run_both(w1, run)
    assert np.array_equal(O1, N1) and np.array_equal(L1, M1)
    g = 3
    ref = oracle_decode(w1, heads=[g])[g]
    gqa = w1["n_head"] // w1["n_head_kv"]
    assert_close(N1[:, g * gqa:(g + 1) * gqa], M1[:, g * gqa:(g + 1) * gqa], *ref, what="noalloc call 1")
    # call 2, smaller: binary16 32/8 heads, 5000 cells, a mask with hidden keys
    w2 = gen.make_workload(1, n_head=32, n_head_kv=8, n_kv=5000, wc=5000)
    rng = np.random.default_rng(3)
    mask = gen.random_mask_f16(rng, 1, w2["n_kv"], p_hidden=0.3)
    step("noalloc call 2: f16 32/8 heads n_kv 5000, mask")
    (O2, L2), (N2, M2) = run_both(w2, run, mask)
    assert np.array_equal(O2, N2) and np.array_equal(L2, M2)
    Oref, Lref = oracle_decode(w2, mask=mask.astype(np.float64))
    assert_close(N2, M2, Oref, Lref, what="noalloc call 2")
    run.ctx.close()


def test_noalloc_fewer_splits_when_the_array_is_full():
    """64 KV heads x 8 query heads each: 512 output rows of 130 floats, so the array holds 31
    partial slots; the persistent binary16 kernel plans one per resident workgroup (more), and
    the entry point runs it with fewer."""
    run = Runner()
    w = gen.make_workload(1, n_head=512, n_head_kv=64, n_kv=8192, wc=8192)
    step("noalloc 512/64 heads n_kv 8192 (split count capped by the static array)")
    (O, L), (N, M) = run_both(w, run)
    Oref, Lref = oracle_decode(w)
    assert_close(N, M, Oref, Lref, what="noalloc capped splits")
    assert_close(O, L, Oref, Lref, what="decode")
    run.ctx.close()


@pytest.mark.parametrize("d,types", [(256, "f16"), (576, "f16"), (64, "q8q4")])
def test_noalloc_other_head_dims_two_calls(d, types):
    """Head dims other than 128 run on their own matrix-core kernels; the entry point plans
    them the same way.  Two calls in a row, the second over fewer cells.  The static array
    may hold fewer partial slots than the context plans here, so the two entry points are
    compared to the fp64 oracle's tolerance rather than bit for bit."""
    run = Runner()
    kt = dict(k_type=gen.TYPE_F16, v_type=gen.TYPE_F16) if types == "f16" else \
        dict(k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    dv = 512 if d == 576 else d
    for n_kv in (6000, 1500):
        w = gen.make_workload(1, d=d, dv=dv, n_head=32, n_head_kv=8, n_kv=n_kv, wc=n_kv, **kt)
        step(f"noalloc {types} d {d} 32/8 heads n_kv {n_kv}")
        (O, L), (N, M) = run_both(w, run)
        Oref, Lref = oracle_decode(w)
        assert_close(N, M, Oref, Lref, what=f"noalloc d {d} n_kv {n_kv}")
        assert_close(O, L, Oref, Lref, what=f"decode d {d} n_kv {n_kv}")
        assert_close(N, M, O.astype(np.float64), L.astype(np.float64), what=f"noalloc vs decode d {d}")
    run.ctx.close()
