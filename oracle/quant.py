"""Oracle: reading stored KV bytes as exact float64 values.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never calls it.

Formats (as stated with the workloads built on the patches' q8_0 K / q4_0 V
caches; the ggml block size of 32 appears in opencoti-llamafile patch
0070-rolling-kv, kv-cache residency hunk, "q8_0 blck 32"):

* f16   : IEEE binary16, little-endian.
* q8_0  : blocks of 34 bytes: binary16 scale ``d`` then 32 signed bytes ``q``;
          element ``i`` of the block is ``d * q[i]``.
* q4_0  : blocks of 18 bytes: binary16 scale ``d`` then 16 bytes; byte ``j``
          holds element ``j`` in its low nibble and element ``j + 16`` in its
          high nibble; element value is ``d * (n - 8)``.

The nibble order is not printed on the pages; the ggml q4_0 layout above is the
reading taken (documented with the other readings of the pages).

Every value is produced in float64, where ``d*q`` and ``d*(n-8)`` are exact.
"""
from __future__ import annotations

import numpy as np

QK = 32


def _scale_f64(blocks: np.ndarray) -> np.ndarray:
    """First two bytes of each block as a little-endian binary16 -> float64."""
    lo = blocks[..., 0].astype(np.uint16)
    hi = blocks[..., 1].astype(np.uint16)
    bits = (lo | (hi << 8)).astype(np.uint16)
    return bits.view(np.float16).astype(np.float64)


def decode_f16(raw: np.ndarray) -> np.ndarray:
    """Bytes (..., 2*n) -> float64 (..., n)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    return raw.view(np.float16).astype(np.float64).reshape(*raw.shape[:-1], raw.shape[-1] // 2)


def decode_q8_0(raw: np.ndarray) -> np.ndarray:
    """Bytes (..., 34*nb) -> float64 (..., 32*nb): element = d * q (q signed)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    nb = raw.shape[-1] // 34
    blk = raw.reshape(*raw.shape[:-1], nb, 34)
    d = _scale_f64(blk)
    q = blk[..., 2:].view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(*raw.shape[:-1], nb * QK)


def decode_q4_0(raw: np.ndarray) -> np.ndarray:
    """Bytes (..., 18*nb) -> float64 (..., 32*nb): element = d * (n - 8)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    nb = raw.shape[-1] // 18
    blk = raw.reshape(*raw.shape[:-1], nb, 18)
    d = _scale_f64(blk)
    packed = blk[..., 2:]
    lo = (packed & 0x0F).astype(np.float64)
    hi = (packed >> 4).astype(np.float64)
    codes = np.concatenate([lo, hi], axis=-1)  # elements 0..15 then 16..31
    return (d[..., None] * (codes - 8.0)).reshape(*raw.shape[:-1], nb * QK)


def decode(type_id: int, raw: np.ndarray) -> np.ndarray:
    if type_id == 1:
        return decode_f16(raw)
    if type_id == 8:
        return decode_q8_0(raw)
    if type_id == 2:
        return decode_q4_0(raw)
    raise ValueError(f"unsupported type {type_id}")
