"""GPU parity of rkv_attn_partial (one segment's (M, S, VKQ) per output row) at head dims 64,
256, 512 and 576/512 against the fp64 oracle's segment partial: q8_0 / q4_0 and binary16
caches, up to 8 rows per KV head (decode kernels) and more (the prefill kernel at 64, the
decode kernels in row groups elsewhere), a segment that starts at a global position with a
causal chunk over it, and an empty segment (opencoti-llamafile patch 0070-rolling-kv: the
per-segment partial that the log-sum-exp combine merges)."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    return Runner()


def call_partial(run, w, seg, kv_pos0, q_pos0):
    import torch
    rkv = run.rkv
    n_q = w["q"].shape[1]
    part = torch.full((n_q * w["n_head"], 2 + w["dv"]), float("nan"), dtype=torch.float32, device="cuda")
    qd = dev(w["q"])
    kd, vd = dev(w["k"][seg]), dev(w["v"][seg])
    run.ctx.attn_partial(rkv.q_desc(qd), rkv.kv_desc(kd, w["k_type"]), rkv.kv_desc(vd, w["v_type"]), None, kv_pos0,
                         q_pos0, w["scale"], part)
    torch.cuda.synchronize()
    return part.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 256, 512, 576])
@pytest.mark.parametrize("types", ["q8q4", "f16"])
@pytest.mark.parametrize("n_q", [1, 6])
def test_partial_head_dims(run, d, types, n_q):
    dv = 512 if d == 576 else d
    kt = dict(k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0) if types == "q8q4" else \
        dict(k_type=gen.TYPE_F16, v_type=gen.TYPE_F16)
    # 32 / 8 heads: 4 rows per KV head at one query, 24 at six
    w = gen.make_workload(1, d=d, dv=dv, n_head=32, n_head_kv=8, n_q=n_q, n_kv=1664, wc=1664, **kt)
    seg = slice(200, 1500)
    q_pos0 = 1400 if n_q > 1 else -1
    step(f"attn_partial d {d}/{dv} {types} n_q {n_q} kv_pos0 200 q_pos0 {q_pos0}")
    P = call_partial(run, w, seg, 200, q_pos0)
    if n_q > 1 and d == 64:
        assert run.ctx.stats()["kernel_variant"] == 1  # the prefill kernel at 64
    qv = oracle.q_values(w["q"])
    kv = oracle.kv_values(w["k_type"], w["k"][seg])
    vv = oracle.kv_values(w["v_type"], w["v"][seg])
    m = oracle.causal_mask(n_q, 1500, q_pos0)[:, 200:1500] if q_pos0 >= 0 else None
    M, S, VKQ = oracle.partial(qv, kv, vv, w["scale"], m)
    # compare as (O = VKQ/S, LSE = M + ln S), the quantities the tolerances are defined on
    Og, Lg = P[:, 2:] / P[:, 1:2], P[:, 0] + np.log(P[:, 1])
    Or, Lr = (VKQ / S[..., None]).reshape(-1, dv), (M + np.log(S)).reshape(-1)
    assert_close(Og, Lg, Or, Lr, what=f"partial d {d}")


@pytest.mark.parametrize("d", [64, 576])
def test_partial_empty_segment(run, d):
    dv = 512 if d == 576 else d
    w = gen.make_workload(1, d=d, dv=dv, n_head=32, n_head_kv=8, n_q=3, n_kv=64, wc=64)
    step(f"attn_partial d {d}/{dv}: empty segment")
    P = call_partial(run, w, slice(0, 0), 0, -1)
    assert np.all(P[:, 0] == -np.inf) and np.all(P[:, 1:] == 0)
