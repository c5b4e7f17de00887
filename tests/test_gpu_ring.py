"""GPU parity of lifted tails through scratch rings of every size (1..4 slots).

With one slot the next tile can only be lifted once the current tile's kernel has read the
slot; with more slots the lift of tile t+1 overlaps tile t.  Each case lifts several tiles,
queues several calls without synchronising between them, and compares every call with the
fp64 oracle."""
import numpy as np
import pytest

import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, pinned, step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_slots", [1, 2, 3, 4])
@pytest.mark.parametrize("layout", ["cell", "head"])
@pytest.mark.parametrize("lift", ["bulk", "kernel"])
def test_ring_sizes(n_slots, layout, lift):
    import torch
    run = Runner()  # a context of its own: the ring size persists on a context
    rkv = run.rkv
    run.ctx.reserve(0, 0, n_slots, 0)
    run.ctx.set_lift_mode(rkv.RKV_LIFT_BULK if lift == "bulk" else rkv.RKV_LIFT_KERNEL)
    w = gen.make_workload(3, scale_down=64)  # n_kv 4096, wc 2048
    wc, tile = 2048, 384  # 6 tiles, the last one ragged
    Oref, Lref = oracle_decode(w)
    kc, vc = w["k"], w["v"]
    if layout == "head":
        kc = np.ascontiguousarray(np.transpose(kc, (1, 0, 2)))
        vc = np.ascontiguousarray(np.transpose(vc, (1, 0, 2)))
        kw, vw, kt, vt = kc[:, :wc], vc[:, :wc], kc[:, wc:], vc[:, wc:]
    else:
        kw, vw, kt, vt = kc[:wc], vc[:wc], kc[wc:], vc[wc:]
    q = dev(w["q"])
    kwd, vwd = dev(np.ascontiguousarray(kw)), dev(np.ascontiguousarray(vw))
    ktp, vtp = pinned(np.ascontiguousarray(kt)), pinned(np.ascontiguousarray(vt))
    junk = torch.randn(2048, 2048, device="cuda")
    outs = []
    step(f"ring {n_slots} slots, {layout}-major tail, {lift} lift, 6 tiles x 3 queued calls")
    for _ in range(3):
        o = torch.empty((1, w["n_head"], 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, w["n_head"]), dtype=torch.float32, device="cuda")
        junk = junk @ junk.T * 1e-3  # unrelated work on the same stream between calls
        run.ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kwd, w["k_type"], layout), rkv.kv_desc(vwd, w["v_type"], layout),
                            rkv.kv_desc(ktp, w["k_type"], layout), rkv.kv_desc(vtp, w["v_type"], layout), None, wc,
                            tile, w["scale"], o, lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    st = run.ctx.stats()
    assert st["n_tail_tiles"] == 6
    for o, lse in outs:
        assert_close(o.cpu().numpy(), lse.cpu().numpy(), Oref, Lref, what=f"ring {n_slots} {layout} {lift}")
    run.ctx.close()
