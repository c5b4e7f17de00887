"""Exact dequantisation where the hot kernels run it, with edge values end to end.

* V: Q = 0 and a mask that leaves one key visible make every softmax weight exactly 1, so O
  must equal that key's dequantised V row bit for bit -- through the matrix-core decode kernel
  (groups of 8, 4 and 2 KV heads), the per-head vector kernel, the head-dim kernel (at 64, 256
  and at 128 for 8 rows per KV head) and the prefill kernel.  The visible V rows hold nibbles 0 and 15 and scales that are zero, negative,
  binary16 subnormal and 65504.
* K: one-hot Q and a single visible key make the LSE equal scale * d * q of one code; rounding
  d*q to binary16 anywhere on the path would move it by ~1e-4 relative, the exact path by
  ~1e-7.  Codes -128 and 127, subnormal and zero scales.
* Random edge bytes (every code and nibble, zero / subnormal / tiny scales) through the same
  kernels against the fp64 oracle at the usual tolerances.
"""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import Runner, assert_close, dev, oracle_decode, step

pytestmark = pytest.mark.gpu

Q8, Q4, F16 = gen.TYPE_Q8_0, gen.TYPE_Q4_0, gen.TYPE_F16
# V block scales (binary16 bits): 1.0, a subnormal, +0, -1.5, 65504, a tiny normal, -0, 0.25
V_SCALES = [0x3C00, 0x0001, 0x0000, 0xBE00, 0x7BFF, 0x0401, 0x8000, 0x3400]


@pytest.fixture(scope="module")
def run():
    return Runner()


def v_edge_row(g, d=128):
    """q4_0 row for KV head g: nibbles cycling through 0..15 (0 and 15 in every block), a
    different scale class per block."""
    blocks = []
    for b in range(d // 32):
        nib = [(3 * e + 5 * g + b) % 16 for e in range(32)]
        nib[0], nib[31] = 0, 15
        blocks.append(gen.block_bytes(Q4, V_SCALES[(4 * g + b) % len(V_SCALES)], nib))
    return np.concatenate(blocks)


def k_edge_row(g, d=128, max_scale_bits=0x5FFF):
    """q8_0 row for KV head g: codes -128, 127 and a spread, scales 0.0999755859375 (d*q needs
    18 significant bits), a subnormal, zero and 65504 (or 25.67 where the path's range ends
    below it)."""
    scales = [0x2E66, 0x0003, 0x0000, 0x7BFF if max_scale_bits >= 0x7BFF else 0x4E6B]
    blocks = []
    for b in range(d // 32):
        codes = [((37 * e + 11 * g + 5 * b) % 256) - 128 for e in range(32)]
        codes[0], codes[1] = -128, 127
        blocks.append(gen.block_bytes(Q8, scales[(g + b) % 4], codes))
    return np.concatenate(blocks)


def edge_workload(n_head, n_head_kv, n_kv, j0, d=128, n_q=1, seed=7, q_zero=True, k_type=Q8, v_type=Q4):
    """Random edge bytes everywhere, the edge rows at key j0, Q zero (or random)."""
    rng = np.random.default_rng(seed)
    k = gen.pack_raw_edge(rng, k_type, (n_kv, n_head_kv), d) if k_type != F16 else \
        gen.pack_f16(rng.standard_normal((n_kv, n_head_kv, d)).astype(np.float32))
    v = gen.pack_raw_edge(rng, v_type, (n_kv, n_head_kv), d) if v_type != F16 else \
        gen.pack_f16(rng.standard_normal((n_kv, n_head_kv, d)).astype(np.float32))
    if v_type == Q4:
        for g in range(n_head_kv):
            v[j0, g] = v_edge_row(g, d)
    q = np.zeros((n_head, n_q, d), np.float16) if q_zero else rng.standard_normal((n_head, n_q, d)).astype(np.float16)
    return dict(q=q, k=k, v=v, k_type=k_type, v_type=v_type, n_head=n_head, n_head_kv=n_head_kv, n_kv=n_kv,
                wc=n_kv, tile_kv=n_kv, scale=1.0, d=d)


def one_key_mask(n_q, n_kv, j0):
    m = np.full((n_q, n_kv), -np.inf, np.float16)
    m[:, j0] = 0
    return m


def expect_v_rows(w, j0):
    """(n_head, d) float32: the dequantised V row of each head's KV head at key j0."""
    gqa = w["n_head"] // w["n_head_kv"]
    vals = oracle.kv_values(w["v_type"], w["v"][j0:j0 + 1])[:, 0]  # (n_head_kv, d)
    return np.repeat(vals, gqa, axis=0).astype(np.float32)


def assert_bits(got, want, what):
    assert np.array_equal(got, want), f"{what}: {np.argwhere(got != want)[:6].tolist()}"
    nz = want != 0
    assert np.array_equal(got[nz].view(np.uint32), want[nz].view(np.uint32)), what


# (name, n_head, n_head_kv, layout, d, expected kernel variant)
DECODE_PATHS = [
    ("decode_mma", 40, 8, "cell", 128, 3),
    ("decode_mma_hw4", 16, 4, "cell", 128, 3),
    ("decode_mma_hw2", 16, 2, "cell", 128, 3),
    ("decode_mma_64", 16, 4, "cell", 64, 3),
    ("decode_mma_64_hw8", 40, 8, "cell", 64, 3),
    ("decode_mma_256", 16, 4, "cell", 256, 3),
    ("decode_mma_256_hw1", 5, 1, "cell", 256, 3),
    ("decode_mma_512", 16, 2, "cell", 512, 3),
    ("vector_head", 16, 4, "head", 128, 0),
    ("head_dim_kernel_at_128", 32, 4, "head", 128, 5),
    ("head_dim_64", 16, 4, "head", 64, 5),
    ("head_dim_256", 16, 4, "head", 256, 5),
]


@pytest.mark.parametrize("name,n_head,n_head_kv,layout,d,variant", DECODE_PATHS)
@pytest.mark.parametrize("tail", [None, "device", "host"])
def test_decode_single_key_v_bit_exact(run, name, n_head, n_head_kv, layout, d, variant, tail):
    n_kv, j0 = 700, 613
    w = edge_workload(n_head, n_head_kv, n_kv, j0, d)
    wc = n_kv if tail is None else 300
    step(f"single-key V exactness: {name} tail {tail}")
    O, L = run.decode(w, wc=wc, tile_kv=256, tail=tail, mask=one_key_mask(1, n_kv, j0), layout=layout)
    assert run.ctx.stats()["kernel_variant"] == variant
    assert_bits(O[0], expect_v_rows(w, j0), f"{name} O")
    assert np.all(L[0] == 0.0)


@pytest.mark.parametrize("tail", [None, "host"])
def test_prefill_single_key_v_bit_exact(run, tail):
    n_kv, j0, n_q = 700, 57, 16
    w = edge_workload(40, 8, n_kv, j0, n_q=n_q)
    step(f"single-key V exactness: prefill tail {tail}")
    O, L = run.decode(w, wc=n_kv if tail is None else 300, tile_kv=256, tail=tail, mask=one_key_mask(n_q, n_kv, j0),
                      prefill=True, q_pos0=-1)
    assert run.ctx.stats()["kernel_variant"] == 1
    want = expect_v_rows(w, j0)
    for i in range(n_q):
        assert_bits(O[i], want, f"prefill O query {i}")
    assert np.all(L == 0.0)


def k_workload(n_head, n_head_kv, n_kv, j0, n_q=1, max_scale_bits=0x5FFF, d=128):
    w = edge_workload(n_head, n_head_kv, n_kv, j0, d=d, n_q=n_q, q_zero=True, v_type=F16)
    for g in range(n_head_kv):
        w["k"][j0, g] = k_edge_row(g, d, max_scale_bits)
    q = np.zeros((n_head, n_q, d), np.float16)
    for h in range(n_head):
        q[h, :, (7 * h + 3) % d] = 1.0  # one-hot: s = d * q of one code
    w["q"] = q
    return w


def check_lse_exact(L, w, mask, what):
    Oref, Lref = oracle_decode(w, mask=np.asarray(mask, np.float64))
    err = np.abs(L - Lref) / np.maximum(np.abs(Lref), 1e-30)
    assert np.all((err <= 2e-6) | (L == Lref)), f"{what}: LSE rel err {err.max():.3e}"


@pytest.mark.parametrize("name,n_head,n_head_kv,layout,d,variant", DECODE_PATHS)
def test_decode_single_key_k_exact(run, name, n_head, n_head_kv, layout, d, variant):
    n_kv, j0 = 500, 333
    w = k_workload(n_head, n_head_kv, n_kv, j0, max_scale_bits=0x7BFF, d=d)
    mask = one_key_mask(1, n_kv, j0)
    step(f"single-key K exactness: {name}")
    O, L = run.decode(w, wc=n_kv, tile_kv=n_kv, tail=None, mask=mask, layout=layout)
    check_lse_exact(L, w, mask, name)


def test_prefill_single_key_k_exact(run):
    """The prefill kernel's two-part K covers |d*q| <= 65504: scales here stay below 512."""
    n_kv, j0, n_q = 500, 333, 8
    w = k_workload(40, 8, n_kv, j0, n_q=n_q)
    mask = one_key_mask(n_q, n_kv, j0)
    step("single-key K exactness: prefill")
    O, L = run.decode(w, wc=n_kv, tile_kv=n_kv, tail=None, mask=mask, prefill=True, q_pos0=-1)
    check_lse_exact(L, w, mask, "prefill")


@pytest.mark.parametrize("name,n_head,n_head_kv,layout,d,variant", DECODE_PATHS)
def test_decode_random_edge_bytes(run, name, n_head, n_head_kv, layout, d, variant):
    """Every code and nibble, zero / subnormal / tiny scales, through the split path."""
    n_kv = 3000
    w = edge_workload(n_head, n_head_kv, n_kv, 0, d=d, seed=11 + d, q_zero=False)
    rng = np.random.default_rng(5)
    mask = gen.random_mask_f16(rng, 1, n_kv, p_hidden=0.2)
    step(f"random edge bytes: {name}")
    O, L = run.decode(w, wc=1700, tile_kv=512, tail="host", mask=mask, layout=layout)
    assert run.ctx.stats()["kernel_variant"] == variant
    Oref, Lref = oracle_decode(w, mask=mask.astype(np.float64))
    assert_close(O, L, Oref, Lref, what=f"edge bytes {name}")


def test_prefill_random_edge_bytes(run):
    n_kv, n_q = 3000, 64
    w = edge_workload(40, 8, n_kv, 0, n_q=n_q, seed=12, q_zero=False)
    step("random edge bytes: prefill causal")
    q_pos0 = n_kv - n_q
    O, L = run.decode(w, wc=1700, tile_kv=512, tail="host", prefill=True, q_pos0=q_pos0)
    Oref, Lref = oracle_decode(w, mask=oracle.causal_mask(n_q, n_kv, q_pos0))
    assert_close(O, L, Oref, Lref, what="edge bytes prefill")


def test_rows_random_edge_bytes(run):
    """Row lists over a q8_0 / q4_0 pool (the per-head vector kernel's row-list form)."""
    rng = np.random.default_rng(13)
    n_pool, n_seq, n_head, n_head_kv = 2000, 3, 16, 4
    k = gen.pack_raw_edge(rng, Q8, (n_pool, n_head_kv), 128)
    v = gen.pack_raw_edge(rng, Q4, (n_pool, n_head_kv), 128)
    rows = gen.rows_lists(rng, n_pool, (700, 1100, 400), 1100)
    mask = np.where(rows[:, None, None, :] >= 0, 0.0, -np.inf).astype(np.float16)
    q = rng.standard_normal((n_seq, n_head, 1, 128)).astype(np.float16)
    w = dict(q=q, k=k, v=v, k_type=Q8, v_type=Q4, kv_rows=rows, mask=mask, scale=1 / np.sqrt(128),
             n_head=n_head, n_head_kv=n_head_kv)
    step("random edge bytes: rows q8_0/q4_0 pool")
    from rkv_testutil import oracle_rows
    O, L = run.rows(w)
    Oref, Lref = oracle_rows(w)
    assert_close(O, L, Oref, Lref, what="edge bytes rows")
