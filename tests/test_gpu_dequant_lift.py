"""Bit-exact checks: the GPU dequantiser against the oracle's reading of the same bytes, and
the tail lift (bulk DMA and the word-granularity contrast) as a byte copy."""
import os

import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import dev, pinned, step

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


FORMS = {"decode_mma": 0, "prefill": 1, "vector": 2, "head_dim": 3}


def gpu_dequant(rows_bytes: np.ndarray, t: int, form: int = 0, row_values: int = 128) -> np.ndarray:
    import torch
    import tiered_kv_cache_split_amd as rkv
    src = dev(rows_bytes)
    dst = torch.empty((rows_bytes.shape[0], row_values), dtype=torch.float32, device="cuda")
    rkv.dequant_rows(src, t, rows_bytes.shape[0], rows_bytes.shape[1], dst, form=form, row_values=row_values)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def assert_exact(got, want):
    """Equal values (a signed zero may come back with either sign) and equal bits otherwise."""
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    nz = want != 0
    assert np.array_equal(got[nz].view(np.uint32), want[nz].view(np.uint32))


def golden_rows(name, block):
    raw = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("bytes "):
            raw.append(bytes.fromhex(line.split()[1]))
    blocks = [np.frombuffer(b, np.uint8) for b in raw]
    while len(blocks) % 4:
        blocks.append(blocks[len(blocks) % len(raw)])
    return np.concatenate(blocks).reshape(-1, 4 * block)


def random_blocks(rng, t, n_rows, row_values, max_abs_scale=65504.0):
    """Raw rows of random bytes: every code / nibble value (q8_0 -128 included) and scales drawn
    from finite binary16 patterns -- zeros of both signs, subnormals, normals up to
    max_abs_scale."""
    nb = row_values // 32
    blk = gen.BLOCK_BYTES[t]
    raw = rng.integers(0, 256, size=(n_rows, nb, blk), dtype=np.uint8)
    bits = rng.integers(0, 1 << 16, size=(n_rows, nb), dtype=np.uint32).astype(np.uint16)
    kind = rng.integers(0, 8, size=(n_rows, nb))
    bits = np.where(kind == 0, bits & 0x8000, bits)                       # +-0
    bits = np.where(kind == 1, bits & 0x83FF, bits)                       # subnormal
    vals = bits.view(np.float16).astype(np.float32)
    bad = ~np.isfinite(vals) | (np.abs(vals) > max_abs_scale)
    bits = np.where(bad, bits & 0x83FF, bits)                             # keep them finite and in range
    raw[..., 0] = (bits & 0xFF).astype(np.uint8)
    raw[..., 1] = (bits >> 8).astype(np.uint8)
    return raw.reshape(n_rows, nb * blk)


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("t", [gen.TYPE_Q8_0, gen.TYPE_Q4_0, gen.TYPE_F16])
def test_dequant_bit_exact_random(t, form):
    """Quantiser output (tiny and all-zero blocks included) through each kernel family's routine."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((4096, 128)).astype(np.float32)
    x[::7] *= 1e-6   # tiny blocks: binary16 subnormal scales
    x[1::97] = 0.0   # all-zero blocks: d = 0
    raw = gen.pack(t, x)
    step(f"dequant type {t} form {form}")
    got = gpu_dequant(raw, t, FORMS[form])
    want = oracle.decode(t, raw).astype(np.float32)
    assert_exact(got, want)


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("t", [gen.TYPE_Q8_0, gen.TYPE_Q4_0])
@pytest.mark.parametrize("row_values", [64, 128, 256])
def test_dequant_bit_exact_raw_bytes(t, form, row_values):
    """Random raw bytes: every code (q8_0 -128 too), nibbles 0 and 15, scales of every binary16
    class up to 65504 (the prefill form's two-part q8_0 operands need |d*q| <= 65504, so its
    scales stay below 511)."""
    rng = np.random.default_rng(1000 + 10 * t + row_values)
    lim = 511.0 if (form == "prefill" and t == gen.TYPE_Q8_0) else 65504.0
    raw = random_blocks(rng, t, 2048, row_values, lim)
    step(f"dequant raw bytes type {t} form {form} d={row_values}")
    got = gpu_dequant(raw, t, FORMS[form], row_values)
    want = oracle.decode(t, raw).astype(np.float32)
    assert_exact(got, want)


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("name,t,blk", [("q8_0_blocks.txt", gen.TYPE_Q8_0, 34), ("q4_0_blocks.txt", gen.TYPE_Q4_0, 18)])
def test_dequant_golden_blocks(name, t, blk, form):
    raw = golden_rows(name, blk)
    step(f"dequant golden {name} form {form}")
    got = gpu_dequant(raw, t, FORMS[form])
    want = oracle.decode(t, raw).astype(np.float32)
    if form == "prefill" and t == gen.TYPE_Q8_0:
        # the two-part binary16 operands cover |d*q| <= 65504 (the scale-65504 block is outside)
        ok = np.abs(want) <= 65504.0
        got, want = got[ok], want[ok]
    assert_exact(got, want)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("nbytes", [1, 4, 8, 4099, 4103, 3 * 1024 * 1024 + 5])
def test_tail_lift_is_a_byte_copy(mode, nbytes):
    import torch
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(nbytes)
    host = pinned(rng.integers(0, 256, size=nbytes, dtype=np.uint8))
    ctx = rkv.Context(0)
    step(f"tail lift mode {mode} nbytes {nbytes}")
    ptr = ctx.tail_lift(host, nbytes, 1, mode)
    torch.cuda.synchronize()
    out = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    assert hip.hipMemcpy(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ptr), ctypes.c_size_t(nbytes), 3) == 0
    assert torch.equal(out.cpu(), host)
    ctx.close()


def test_pageable_tail_is_rejected():
    import torch
    import tiered_kv_cache_split_amd as rkv
    w = gen.make_workload(1)
    ctx = rkv.Context(0)
    q = dev(w["q"])
    kw, vw = dev(w["k"][:2048]), dev(w["v"][:2048])
    kt = torch.from_numpy(np.ascontiguousarray(w["k"][2048:]))  # pageable
    vt = torch.from_numpy(np.ascontiguousarray(w["v"][2048:]))
    o = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(rkv.RkvError) as e:
        ctx.attn_decode(rkv.q_desc(q), rkv.kv_desc(kw, 1), rkv.kv_desc(vw, 1), rkv.kv_desc(kt, 1),
                        rkv.kv_desc(vt, 1), None, 2048, 1024, 0.088, o)
    assert e.value.status == -1
    ctx.close()
