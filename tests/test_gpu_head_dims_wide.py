"""Head dim 512 (dk = dv) and the dk = 576 / dv = 512 pair through rkv_attn_decode and
rkv_lse_merge against the fp64 oracle, as the streaming op of opencoti-llamafile patch
0070-rolling-kv lists them among its shapes (fattn.cu, the op's supported head dims): the window
+ tail split with a lifted (both engines) or device-resident tail, every K/V type pair, masks
with an empty row, the soft-cap, grouped-query rows up to eight per KV head, the empty cache,
exact single-key V and one-hot K, the tail's partial on the host cores; unsupported pairs are
refused."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu

PAIRS = [(gen.TYPE_F16, gen.TYPE_F16), (gen.TYPE_Q8_0, gen.TYPE_Q4_0), (gen.TYPE_Q8_0, gen.TYPE_F16),
         (gen.TYPE_F16, gen.TYPE_Q4_0)]
DIMS = [(512, 512), (576, 512)]


@pytest.fixture(scope="module")
def run():
    r = Runner()
    yield r
    r.ctx.set_lift_mode(r.rkv.RKV_LIFT_AUTO)
    r.ctx.set_softcap(0.0)
    r.ctx.set_tail_mode(r.rkv.RKV_TAIL_LIFT)


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("kt,vt", PAIRS)
@pytest.mark.parametrize("lift", [0, 2])
def test_window_plus_lifted_tail(run, dk, dv, kt, vt, lift):
    w = gen.make_workload(1, d=dk, dv=dv, k_type=kt, v_type=vt)  # 8/2 heads, n_kv 4096
    run.ctx.set_lift_mode(lift)
    step(f"head dims {dk}/{dv}: k={kt} v={vt} wc=1333 tile=700 lift {lift}")
    O, L = run.decode(w, wc=1333, tile_kv=700, tail="host")
    st = run.ctx.stats()
    # q8_0 / q4_0 (512 / 512 and 576 / 512): the matrix-core kernel; binary16 (two KV heads: one
    # cell group at 512, two groups of one at 576): the binary16 matrix-core kernel; mixed: vector
    mma = (kt, vt) == (gen.TYPE_Q8_0, gen.TYPE_Q4_0)
    mma16 = (kt, vt) == (gen.TYPE_F16, gen.TYPE_F16)
    assert st["kernel_variant"] == (3 if mma else 4 if mma16 else 5) and st["n_tail_tiles"] == -(-(4096 - 1333) // 700)
    assert O.shape == (1, 8, dv)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv}")


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("layout", ["cell", "head"])
def test_device_tail_and_layouts(run, dk, dv, layout):
    w = gen.make_workload(3, scale_down=64, d=dk, dv=dv)  # q8_0 K, q4_0 V, 40/8 heads, n_kv 4096
    step(f"head dims {dk}/{dv}: q8q4 layout {layout} device tail")
    O, L = run.decode(w, tail="device", layout=layout)
    Oref, Lref = oracle_decode(w)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} {layout}")
    run.ctx.set_lift_mode(run.rkv.RKV_LIFT_KERNEL)
    step(f"head dims {dk}/{dv}: q8q4 layout {layout} lifted tail, copy kernel")
    O, L = run.decode(w, tail="host", layout=layout)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} {layout} lifted")


@pytest.mark.parametrize("dk,dv", DIMS)
@pytest.mark.parametrize("n_head,n_head_kv,n_q", [(8, 2, 2), (16, 2, 1), (8, 1, 1)])
def test_mask_gqa_and_empty_row(run, dk, dv, n_head, n_head_kv, n_q):
    w = gen.make_workload(1, d=dk, dv=dv, n_q=n_q, n_head=n_head, n_head_kv=n_head_kv,
                          k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    mask = gen.random_mask_f16(np.random.default_rng(dk + n_head), n_q, w["n_kv"], p_hidden=0.4)
    mask[n_q - 1, :] = -np.inf  # the last query sees nothing
    step(f"head dims {dk}/{dv}: mask, heads {n_head}/{n_head_kv}, n_q {n_q}")
    O, L = run.decode(w, wc=2000, tile_kv=1024, tail="host", mask=mask)
    Oref, Lref = oracle_decode(w, mask=mask)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} mask")
    assert np.all(O[n_q - 1] == 0) and np.all(L[n_q - 1] == -np.inf)


@pytest.mark.parametrize("dk,dv", DIMS)
def test_softcap_and_outliers(run, dk, dv):
    w = gen.make_workload(2, scale_down=32, d=dk, dv=dv)  # q8q4, 40/8 heads, n_kv 4096
    run.ctx.set_softcap(30.0)
    try:
        step(f"head dims {dk}/{dv}: soft-cap 30, window 2500 + lifted tail")
        O, L = run.decode(w, wc=2500, tile_kv=512, tail="host")
    finally:
        run.ctx.set_softcap(0.0)
    Oref, Lref = oracle_decode(w, softcap=30.0)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} softcap")


@pytest.mark.parametrize("dk,dv", DIMS)
def test_whole_cache_in_the_tail_and_window_only(run, dk, dv):
    w = gen.make_workload(1, d=dk, dv=dv, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    Oref, Lref = oracle_decode(w)
    step(f"head dims {dk}/{dv}: wc = 0")
    O, L = run.decode(w, wc=0, tile_kv=999, tail="host")
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} wc=0")
    step(f"head dims {dk}/{dv}: window only")
    O, L = run.decode(w, wc=w["n_kv"], tail=None)
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} window only")


@pytest.mark.parametrize("dk,dv", DIMS)
def test_empty_cache(dk, dv):
    import torch
    import tiered_kv_cache_split_amd as rkv
    ctx = rkv.Context(0)
    try:
        q = dev(np.random.default_rng(3).standard_normal((8, 1, dk)).astype(np.float16))
        kw = torch.empty((0, 2, 2 * dk), dtype=torch.uint8, device="cuda")
        vw = torch.empty((0, 2, 2 * dv), dtype=torch.uint8, device="cuda")
        o = torch.full((1, 8, dv), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
        step(f"head dims {dk}/{dv}: n_kv = 0")
        ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kw, gen.TYPE_F16), rkv.kv_desc(vw, gen.TYPE_F16), None, None,
                        None, 0, 64, 0.04, o, lse)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(lse == -float("inf"))
    finally:
        ctx.close()


def q4_row(rng, dv, scales):
    """q4_0 row of dv values: nibbles with 0 and 15 in every block, the given scales (bits)."""
    blocks = []
    for b in range(dv // 32):
        nib = list(rng.integers(0, 16, 32))
        nib[0], nib[31] = 0, 15
        blocks.append(gen.block_bytes(gen.TYPE_Q4_0, scales[b % len(scales)], nib))
    return np.concatenate(blocks)


@pytest.mark.parametrize("dk,dv", DIMS)
def test_single_key_v_bit_exact(run, dk, dv):
    """Q = 0 and one visible key: every weight is exactly 1, so O equals that key's dequantised
    V row bit for bit (scales 1, subnormal, 0, -1.5, 65504, tiny, -0, 0.25)."""
    rng = np.random.default_rng(dk)
    n_kv, j0 = 900, 611
    w = gen.make_workload(1, d=dk, dv=dv, n_head=8, n_head_kv=2, k_type=gen.TYPE_Q8_0, v_type=gen.TYPE_Q4_0)
    w["n_kv"] = n_kv
    w["k"], w["v"] = w["k"][:n_kv].copy(), w["v"][:n_kv].copy()
    for g in range(2):
        w["v"][j0, g] = q4_row(rng, dv, [0x3C00, 0x0001, 0x0000, 0xBE00, 0x7BFF, 0x0401, 0x8000, 0x3400])
    w["q"] = np.zeros_like(w["q"])
    mask = np.full((1, n_kv), -np.inf, np.float16)
    mask[0, j0] = 0
    step(f"head dims {dk}/{dv}: single-key V exactness")
    O, L = run.decode(w, wc=500, tile_kv=256, tail="host", mask=mask)
    want = np.repeat(oracle.kv_values(gen.TYPE_Q4_0, w["v"][j0:j0 + 1])[:, 0], 4, axis=0).astype(np.float32)
    assert np.array_equal(O[0], want)
    nz = want != 0
    assert np.array_equal(O[0][nz].view(np.uint32), want[nz].view(np.uint32))
    assert np.all(L[0] == 0.0)


@pytest.mark.parametrize("vt", [gen.TYPE_F16, gen.TYPE_Q4_0])
def test_one_hot_k_exact_at_576(vt):
    """dk = 576: one-hot Q on each of the last two blocks' dims and on a main block, one visible
    key: the LSE is scale * d * q of one code (codes -128 / 127, scales needing 11 bits); binary16
    V runs on the vector kernel, q4_0 V on the matrix-core kernel."""
    run = Runner()
    rng = np.random.default_rng(576)
    n_kv, j0 = 300, 123
    w = gen.make_workload(1, d=576, dv=512, n_head=8, n_head_kv=2, k_type=gen.TYPE_Q8_0, v_type=vt)
    w["n_kv"] = n_kv
    w["k"], w["v"] = w["k"][:n_kv].copy(), w["v"][:n_kv].copy()
    for g in range(2):
        blocks = []
        for b in range(18):
            codes = list(rng.integers(-128, 128, 32))
            codes[0], codes[31] = -128, 127
            blocks.append(gen.block_bytes(gen.TYPE_Q8_0, 0x2E66 + 7 * b, codes))
        w["k"][j0, g] = np.concatenate(blocks)
    q = np.zeros_like(w["q"])
    for h, dim in enumerate([512, 543, 544, 575, 0, 31, 300, 511]):
        q[h, :, dim] = 1.0
    w["q"] = q
    mask = np.full((1, n_kv), -np.inf, np.float16)
    mask[0, j0] = 0
    step(f"head dims 576/512: one-hot K exactness, V type {vt}")
    O, L = run.decode(w, wc=200, tile_kv=64, tail="host", mask=mask)
    assert run.ctx.stats()["kernel_variant"] == (3 if vt == gen.TYPE_Q4_0 else 5)
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    err = np.abs(L - Lref) / np.maximum(np.abs(Lref), 1e-30)
    assert np.all((err <= 2e-6) | (L == Lref)), err.max()
    run.ctx.close()


def test_lse_merge_dv512():
    import torch
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(512)
    H, G, N, dk, dv = 8, 2, 300, 576, 512
    q = rng.standard_normal((H, 1, dk))
    k = rng.standard_normal((G, N, dk))
    v = rng.standard_normal((G, N, dv))
    bounds = [0, 100, 100, 217, 300]
    parts = [oracle.partial(q, k[:, a:b], v[:, a:b], 0.04) for a, b in zip(bounds, bounds[1:])]
    buf = np.zeros((len(parts), H, 2 + dv), dtype=np.float32)
    for s_, (M, S, VKQ) in enumerate(parts):
        buf[s_, :, 0] = M.reshape(-1)
        buf[s_, :, 1] = S.reshape(-1)
        buf[s_, :, 2:] = VKQ.reshape(H, dv)
    o = torch.empty((H, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((H,), dtype=torch.float32, device="cuda")
    step("lse merge dv 512")
    rkv.lse_merge(dev(buf), len(parts), H, o, lse, dv=dv)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(q, k, v, 0.04)
    assert_close(o.cpu().numpy()[None], lse.cpu().numpy()[None], Oref.reshape(1, H, dv), Lref.reshape(1, H),
                 what="merge dv=512")


def test_refusals(run):
    import torch
    rkv = run.rkv
    step("head dims: unsupported pairs refused")
    for dk, dv in [(576, 576), (512, 576), (512, 256), (576, 128)]:
        w = gen.make_workload(1, d=dk, dv=dv, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16)
        with pytest.raises(rkv.RkvError) as e:
            run.decode(w, wc=2048, tile_kv=1024, tail="host")
        assert e.value.status in (rkv.RKV_ERR_UNSUPPORTED, rkv.RKV_ERR_ARG), (dk, dv)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dk,dv", DIMS)
def test_host_tail_partial(run, dk, dv):
    """The tail's partial on the host cores (RKV_TAIL_HOST), merged with the window's."""
    rkv = run.rkv
    w = gen.make_workload(3, scale_down=64, d=dk, dv=dv)  # q8q4, 40/8 heads, n_kv 4096, wc 2048
    mask = gen.random_mask_f16(np.random.default_rng(dk), 1, w["n_kv"], p_hidden=0.3)
    run.ctx.set_tail_mode(rkv.RKV_TAIL_HOST)
    try:
        step(f"head dims {dk}/{dv}: host tail partial with a mask")
        O, L = run.decode(w, tail="host", mask=mask)
        assert run.ctx.stats()["tail_host"] == 1
    finally:
        run.ctx.set_tail_mode(rkv.RKV_TAIL_LIFT)
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    assert_close(O, L, Oref, Lref, what=f"d={dk}/{dv} host tail")
