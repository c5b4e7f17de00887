"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only *draws* inputs and packs them into bytes.  It holds none of the
method's arithmetic: no attention, no softmax, no merge and no dequantisation.
Both sides of every parity check (the fp64 oracle and the HIP library) read the
same bytes produced here and decode them independently.

Value recipe (stated once, used everywhere):
  * numpy ``Generator(PCG64(seed))``; seed = 20261200 + workload number;
  * draws happen in the order Q, then K, then V, iid N(0, 1) in float32;
  * f16 tensors are the float32 draws rounded to IEEE binary16 (round to nearest even);
  * q8_0 / q4_0 tensors are the float32 draws quantised per 32-value block
    (formats below).

Block formats (32 values per block, little-endian, the scale stored first):
  * q8_0: 34 bytes = binary16 scale ``d`` + 32 signed bytes ``q``; value ``d*q``.
  * q4_0: 18 bytes = binary16 scale ``d`` + 16 bytes of nibbles; byte ``j`` holds
    element ``j`` in its low nibble and element ``j+16`` in its high nibble;
    value ``d*(n-8)``.

The quantisers below only generate input bytes; how the bytes are *read* is
defined independently in ``oracle/quant.py`` and in the HIP dequantiser.

Tensor layouts follow the ggml convention of the pages (``ne[0]`` fastest):
  * Q ``[d, n_q, n_head]`` -> numpy array of shape ``(n_head, n_q, d)``;
  * K/V caches are stored *cell-major* (all KV heads of one cell together):
    numpy uint8 array of shape ``(n_cells, n_head_kv, row_bytes)``;
  * mask ``[n_kv, n_q]`` -> numpy float16 ``(n_q, n_kv)`` (additive, -inf = hidden).
"""
from __future__ import annotations

import numpy as np

QK = 32  # values per quant block
TYPE_F32, TYPE_F16, TYPE_Q4_0, TYPE_Q8_0 = 0, 1, 2, 8
BLOCK_BYTES = {TYPE_Q8_0: 34, TYPE_Q4_0: 18}
TYPE_NAMES = {TYPE_F32: "f32", TYPE_F16: "f16", TYPE_Q4_0: "q4_0", TYPE_Q8_0: "q8_0"}
SEED_BASE = 20261200


def rng_for(workload: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(SEED_BASE + int(workload)))


def row_bytes(type_id: int, d: int) -> int:
    if type_id == TYPE_F16:
        return 2 * d
    if type_id == TYPE_F32:
        return 4 * d
    assert d % QK == 0
    return (d // QK) * BLOCK_BYTES[type_id]


def values_per_row(type_id: int, n_bytes: int) -> int:
    """Values in a row of n_bytes bytes of the given type (the inverse of row_bytes)."""
    if type_id == TYPE_F16:
        return n_bytes // 2
    if type_id == TYPE_F32:
        return n_bytes // 4
    assert n_bytes % BLOCK_BYTES[type_id] == 0
    return n_bytes // BLOCK_BYTES[type_id] * QK


# ---------------------------------------------------------------- packers
def pack_f16(x: np.ndarray) -> np.ndarray:
    """float32 values -> raw binary16 bytes (last axis becomes 2*len)."""
    h = np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    return h.view(np.uint8).reshape(*x.shape[:-1], 2 * x.shape[-1])


def pack_q8_0(x: np.ndarray) -> np.ndarray:
    """float32 values (last axis a multiple of 32) -> q8_0 bytes.

    Scale ``d = amax/127`` per block (stored as binary16), codes
    ``q = clip(rint(x/d), -127, 127)``; an all-zero block gets ``d = 0``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead, n = x.shape[:-1], x.shape[-1]
    assert n % QK == 0
    b = x.reshape(-1, QK)
    amax = np.abs(b).max(axis=1)
    d = (amax / 127.0).astype(np.float32)
    inv = np.where(d > 0, 1.0 / np.where(d > 0, d, 1), 0.0).astype(np.float32)
    q = np.clip(np.rint(b * inv[:, None]), -127, 127).astype(np.int8)
    out = np.empty((b.shape[0], 34), dtype=np.uint8)
    out[:, 0:2] = d.astype(np.float16).reshape(-1, 1).view(np.uint8)
    out[:, 2:] = q.view(np.uint8)
    return out.reshape(*lead, (n // QK) * 34)


def pack_q4_0(x: np.ndarray) -> np.ndarray:
    """float32 values (last axis a multiple of 32) -> q4_0 bytes.

    ``m`` is the block element of largest magnitude (sign kept), ``d = m/-8``
    (stored as binary16), codes ``n = clip(floor(x/d + 8.5), 0, 15)``; byte ``j``
    packs element ``j`` (low nibble) and element ``j+16`` (high nibble)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead, n = x.shape[:-1], x.shape[-1]
    assert n % QK == 0
    b = x.reshape(-1, QK)
    idx = np.abs(b).argmax(axis=1)
    m = b[np.arange(b.shape[0]), idx]
    d = (m / -8.0).astype(np.float32)
    inv = np.where(d != 0, 1.0 / np.where(d != 0, d, 1), 0.0).astype(np.float32)
    codes = np.clip(np.floor(b * inv[:, None] + 8.5), 0, 15).astype(np.uint8)
    out = np.empty((b.shape[0], 18), dtype=np.uint8)
    out[:, 0:2] = d.astype(np.float16).reshape(-1, 1).view(np.uint8)
    out[:, 2:] = codes[:, :16] | (codes[:, 16:] << 4)
    return out.reshape(*lead, (n // QK) * 18)


def pack(type_id: int, x: np.ndarray) -> np.ndarray:
    if type_id == TYPE_F16:
        return pack_f16(x)
    if type_id == TYPE_Q8_0:
        return pack_q8_0(x)
    if type_id == TYPE_Q4_0:
        return pack_q4_0(x)
    raise ValueError(f"unsupported type {type_id}")


def pack_raw_edge(rng, type_id: int, lead_shape, d: int, p_zero=0.1, p_sub=0.1, p_tiny=0.1,
                  scale_sigma=1.0 / 64) -> np.ndarray:
    """Raw q8_0 / q4_0 rows of random bytes for edge coverage: every code byte (q8_0 -128
    included) and every nibble (0 and 15 included) equally likely; block scales drawn as
    binary16 bit patterns: +-0 with probability p_zero, a subnormal with p_sub, a tiny normal
    (< 2**-10) with p_tiny, otherwise |N(0, scale_sigma)| with a random sign.  Shape
    lead_shape + (row_bytes,)."""
    lead = tuple(lead_shape)
    nb = d // QK
    blk = BLOCK_BYTES[type_id]
    raw = rng.integers(0, 256, size=lead + (nb, blk), dtype=np.uint8)
    normal = (rng.standard_normal(lead + (nb,)) * scale_sigma).astype(np.float16).view(np.uint16)
    u = rng.random(lead + (nb,))
    sign = rng.integers(0, 2, size=lead + (nb,)).astype(np.uint16) << 15
    sub = (rng.integers(1, 1 << 10, size=lead + (nb,)).astype(np.uint16)) | sign
    tiny = (rng.integers(1 << 10, 6 << 10, size=lead + (nb,)).astype(np.uint16)) | sign
    bits = np.where(u < p_zero, sign, np.where(u < p_zero + p_sub, sub, np.where(u < p_zero + p_sub + p_tiny, tiny, normal)))
    raw[..., 0] = (bits & 0xFF).astype(np.uint8)
    raw[..., 1] = (bits >> 8).astype(np.uint8)
    return raw.reshape(lead + (nb * blk,))


def block_bytes(type_id: int, scale_bits: int, codes) -> np.ndarray:
    """One q8_0 block (codes: 32 ints in [-128, 127]) or q4_0 block (codes: 32 nibbles in
    [0, 15], element order) as bytes, with the given binary16 scale bit pattern."""
    c = np.asarray(codes, dtype=np.int64)
    assert c.shape == (QK,)
    out = np.empty(BLOCK_BYTES[type_id], dtype=np.uint8)
    out[0], out[1] = scale_bits & 0xFF, (scale_bits >> 8) & 0xFF
    if type_id == TYPE_Q8_0:
        out[2:] = (c & 0xFF).astype(np.uint8)
    else:
        out[2:] = (c[:16] | (c[16:] << 4)).astype(np.uint8)
    return out


# ---------------------------------------------------------------- draws
def draw_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def draw_qkv(rng, n_head, n_q, n_head_kv, n_kv, d=128, dv=128, k_type=TYPE_F16,
             v_type=TYPE_F16, outlier_every=0, outlier_scale=30.0):
    """Q as f16 values ``(n_head, n_q, d)``; K/V as cell-major byte caches
    ``(n_kv, n_head_kv, row_bytes)``.  With ``outlier_every=m`` every m-th
    cell's K is multiplied by ``outlier_scale`` before packing."""
    q = draw_normal(rng, (n_head, n_q, d)).astype(np.float16)
    k = draw_normal(rng, (n_kv, n_head_kv, d))
    v = draw_normal(rng, (n_kv, n_head_kv, dv))
    if outlier_every:
        k[::outlier_every] *= np.float32(outlier_scale)
    return q, pack(k_type, k), pack(v_type, v)


def causal_mask_f16(n_q: int, n_kv: int, q_pos0: int) -> np.ndarray:
    """Additive f16 mask (n_q, n_kv): query i at position q_pos0+i sees keys <= it."""
    j = np.arange(n_kv)[None, :]
    i = np.arange(n_q)[:, None] + q_pos0
    return np.where(j <= i, 0.0, -np.inf).astype(np.float16)


def random_mask_f16(rng, n_q: int, n_kv: int, p_hidden=0.3, with_bias=True) -> np.ndarray:
    """Random additive mask: hidden entries -inf, visible ones 0 or a small bias."""
    hid = rng.random((n_q, n_kv)) < p_hidden
    bias = (rng.standard_normal((n_q, n_kv)) * 0.5) if with_bias else np.zeros((n_q, n_kv))
    return np.where(hid, -np.inf, bias).astype(np.float16)


# ---------------------------------------------------------------- workloads
WORKLOADS = {
    1: dict(name="decode_f16_win2048_tail2048", kind="decode", n_head=8, n_head_kv=2, d=128,
            n_q=1, n_kv=4096, wc=2048, tile_kv=1024, k_type=TYPE_F16, v_type=TYPE_F16),
    2: dict(name="decode_q8q4_nkv131072_resident", kind="decode", n_head=40, n_head_kv=8, d=128,
            n_q=1, n_kv=131072, wc=131072, tile_kv=32768, k_type=TYPE_Q8_0, v_type=TYPE_Q4_0),
    3: dict(name="decode_q8q4_win131072_tail131072", kind="decode", n_head=40, n_head_kv=8,
            d=128, n_q=1, n_kv=262144, wc=131072, tile_kv=32768, k_type=TYPE_Q8_0,
            v_type=TYPE_Q4_0),
    4: dict(name="rows_f16_pool65536_4seq", kind="rows", n_head=32, n_head_kv=8, d=128, n_q=1,
            n_pool=65536, lengths=(8192, 12288, 20480, 30720), n_kv=30720, k_type=TYPE_F16,
            v_type=TYPE_F16),
    5: dict(name="prefill_q8q4_nq512_nkv106496", kind="prefill", n_head=40, n_head_kv=8, d=128,
            n_q=512, n_kv=106496, wc=65536, tile_kv=32768, q_pos0=106496 - 512,
            k_type=TYPE_Q8_0, v_type=TYPE_Q4_0),
}


def rows_lists(rng, n_pool: int, lengths, n_kv_pad: int, shuffle=False) -> np.ndarray:
    """Row lists for the unified-pool workload, shape (n_seq, n_kv_pad) int32.

    One seeded permutation of the pool; sequence b takes the next ``lengths[b]``
    entries of it (wrapping round, so lists are disjoint while the pool lasts
    and overlap only once it is exhausted); rows are unique within a list and
    sorted ascending unless ``shuffle``; padding is -1."""
    perm = rng.permutation(n_pool).astype(np.int64)
    out = np.full((len(lengths), n_kv_pad), -1, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lengths):
        idx = (pos + np.arange(L)) % n_pool
        r = perm[idx]
        pos += L
        r = rng.permutation(r) if shuffle else np.sort(r)
        out[b, :L] = r
    return out


def make_workload(num: int, scale_down: int = 1, **over):
    """Draw the inputs of a workload.  ``scale_down`` divides the KV lengths
    (window, tail, tile, pool, list lengths) for oracle-sized variants."""
    w = dict(WORKLOADS[num])
    w.update(over)
    rng = rng_for(num)
    sd = max(1, int(scale_down))
    if w["kind"] == "rows":
        n_pool = w["n_pool"] // sd
        lengths = tuple(max(1, L // sd) for L in w["lengths"])
        n_kv = max(lengths)
        n_seq = len(lengths)
        dv = w.get("dv", w["d"])
        q = draw_normal(rng, (n_seq, w["n_head"], w["n_q"], w["d"])).astype(np.float16)
        k = pack(w["k_type"], draw_normal(rng, (n_pool, w["n_head_kv"], w["d"])))
        v = pack(w["v_type"], draw_normal(rng, (n_pool, w["n_head_kv"], dv)))
        rows = rows_lists(rng, n_pool, lengths, n_kv)
        mask = np.where(rows[:, None, None, :] >= 0, 0.0, -np.inf).astype(np.float16)
        mask = np.broadcast_to(mask, (n_seq, 1, w["n_q"], n_kv)).copy()
        w.update(n_pool=n_pool, lengths=lengths, n_kv=n_kv, n_seq=n_seq)
        w.update(q=q, k=k, v=v, kv_rows=rows, mask=mask, scale=1.0 / np.sqrt(w["d"]), dv=dv)
        return w
    n_kv = w["n_kv"] // sd
    wc = min(n_kv, w["wc"] // sd)
    tile = max(1, w["tile_kv"] // sd)
    dv = w.get("dv", w["d"])  # V head dim (differs from Q/K's only in the 576/512 pair)
    q, k, v = draw_qkv(rng, w["n_head"], w["n_q"], w["n_head_kv"], n_kv, w["d"], dv,
                       w["k_type"], w["v_type"])
    w.update(n_kv=n_kv, wc=wc, tile_kv=tile, q=q, k=k, v=v, scale=1.0 / np.sqrt(w["d"]),
             mask=None, dv=dv)
    if w["kind"] == "prefill":
        w["q_pos0"] = n_kv - w["n_q"]
    return w
