"""Oracle: plain float64 softmax attention, segment partials and their merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library: inputs arrive as the same raw bytes, decoded by
``oracle/quant.py``.

What is computed (for query ``i``, head ``h``; KV head ``g = h // (n_head/n_head_kv)``,
query heads sharing a KV head being contiguous as in the grouped-query mapping
of opencoti-llamafile patch 0070-rolling-kv, fattn.cu ``streaming_lse_kernel``):

    s_j   = scale * <q_{i,h}, k_{j,g}> + mask[i, j]           (mask additive, -inf hides)
    V     = { j : s_j > -inf }
    LSE   = ln sum_{j in V} exp(s_j)
    O     = sum_{j in V} exp(s_j - LSE) * v_{j,g}
    V empty  ->  O = 0, LSE = -inf

The scale is applied before the mask (patch 0070, fattn.cu ``streaming_lse_kernel``:
``scale*part`` then ``+= mask``; a -inf key contributes nothing; ``lse = m + log l``
or -inf when ``l = 0``).  With a logit soft-cap ``c > 0`` the scaled score is
replaced, still before the mask, by ``c * tanh(scale * <q, k> / c)`` (the same
kernel's soft-cap branch); ``c = 0`` is the plain score.

A *segment partial* over a subset of key positions is ``(M, S, VKQ)``:
``M = max s_j``, ``S = sum exp(s_j - M)``, ``VKQ = sum exp(s_j - M) v_j``
(patch 0070, ``ggml_flash_attn_ext_tail_partial`` and
``tail_partial_to_tile_kernel``: ``[M, S, VKQ_unnorm]`` per output row, ``O = VKQ/S``,
``lse = M + log S``).  The merge of partials is the log-sum-exp combine of patch
0070's fattn.cu header comment and ``streaming_combine_kernel``:
``M* = max M``, ``S* = sum S e^(M - M*)``, ``VKQ* = sum VKQ e^(M - M*)``,
``O = VKQ*/S*``, ``LSE = M* + ln S*``; an empty segment has weight 0.

The unified-pool variant follows llama.cpp PR #29510 (``ggml_flash_attn_ext_rows``
API comment): key ``j`` of sequence ``b`` is pool row ``kv_rows[b, j]``; a negative
row is padding and contributes nothing (it is never dereferenced).

numpy's matmul / exp / log serve as library primitives; everything is float64.
"""
from __future__ import annotations

import numpy as np

from .quant import decode

NEG_INF = -np.inf


def kv_values(type_id: int, cache: np.ndarray) -> np.ndarray:
    """Cell-major cache bytes (n_cells, n_head_kv, row_bytes) -> (n_head_kv, n_cells, d) f64."""
    vals = decode(type_id, cache)  # (n_cells, n_head_kv, d)
    return np.ascontiguousarray(np.transpose(vals, (1, 0, 2)))


def q_values(q_f16: np.ndarray) -> np.ndarray:
    return np.asarray(q_f16, dtype=np.float16).astype(np.float64)


def scores(q, k, scale, mask=None, softcap=0.0):
    """q (n_head, n_q, d), k (n_head_kv, n, d), mask (n_q, n) or None -> s (n_head, n_q, n)."""
    n_head = q.shape[0]
    n_head_kv = k.shape[0]
    assert n_head % n_head_kv == 0
    gqa = n_head // n_head_kv
    s = np.empty((n_head, q.shape[1], k.shape[1]), dtype=np.float64)
    for h in range(n_head):
        g = h // gqa
        s[h] = scale * (q[h] @ k[g].T)
    if softcap:
        s = softcap * np.tanh(s / softcap)
    if mask is not None:
        s = s + np.asarray(mask, dtype=np.float64)[None, :, :]
    return s


def partial(q, k, v, scale, mask=None, softcap=0.0):
    """Segment partial over all keys given: returns M, S (n_q, n_head) and VKQ (n_q, n_head, dv)."""
    s = scores(q, k, scale, mask, softcap)  # (n_head, n_q, n)
    n_head, n_q, n = s.shape
    gqa = n_head // k.shape[0]
    dv = v.shape[2]
    M = np.full((n_q, n_head), NEG_INF)
    S = np.zeros((n_q, n_head))
    VKQ = np.zeros((n_q, n_head, dv))
    if n == 0:
        return M, S, VKQ
    vis = s > NEG_INF
    any_vis = vis.any(axis=2)  # (n_head, n_q)
    m = np.where(any_vis, np.where(vis, s, NEG_INF).max(axis=2), 0.0)
    e = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[:, :, None]), 0.0)
    for h in range(n_head):
        VKQ[:, h, :] = e[h] @ v[h // gqa]
    M[:, :] = np.where(any_vis, m, NEG_INF).T
    S[:, :] = e.sum(axis=2).T
    return M, S, VKQ


def merge(parts):
    """Log-sum-exp merge of a list of (M, S, VKQ) partials -> O (n_q, n_head, dv), LSE (n_q, n_head)."""
    Ms = np.stack([p[0] for p in parts])
    Mstar = Ms.max(axis=0)
    finite = Mstar > NEG_INF
    Ssum = np.zeros_like(Mstar)
    Vsum = np.zeros_like(parts[0][2])
    for M, S, VKQ in parts:
        w = np.where((M > NEG_INF) & finite, np.exp(np.where(M > NEG_INF, M, 0.0) -
                                                     np.where(finite, Mstar, 0.0)), 0.0)
        Ssum += S * w
        Vsum += VKQ * w[..., None]
    ok = finite & (Ssum > 0)
    O = np.where(ok[..., None], Vsum / np.where(ok, Ssum, 1.0)[..., None], 0.0)
    LSE = np.where(ok, np.where(ok, Mstar, 0.0) + np.log(np.where(ok, Ssum, 1.0)), NEG_INF)
    return O, LSE


def attention(q, k, v, scale, mask=None, softcap=0.0):
    """Unsplit attention over all keys: O (n_q, n_head, dv), LSE (n_q, n_head)."""
    return merge([partial(q, k, v, scale, mask, softcap)])


def split_attention(q, k, v, scale, mask, bounds, softcap=0.0):
    """Attention computed as partials over the position segments [b_t, b_{t+1}) then merged."""
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        parts.append(partial(q, k[:, a:b], v[:, a:b], scale,
                             None if mask is None else mask[:, a:b], softcap))
    return merge(parts)


def window_tail_bounds(n_kv: int, wc: int, tile_kv: int):
    """Position segments of a device window [0, wc) plus a tail [wc, n_kv) cut into
    tiles of tile_kv keys, none straddling wc (patch 0070, fattn.cu ``resolve(t)``:
    window and tail are tiled separately; a tail tile's global offset is wc + local)."""
    b = [0]
    if wc > 0:
        b.append(wc)
    t = wc
    while t < n_kv:
        t = min(n_kv, t + tile_kv)
        b.append(t)
    return b


def causal_mask(n_q: int, n_kv: int, q_pos0: int) -> np.ndarray:
    """Explicit additive mask (n_q, n_kv): query i at absolute position q_pos0 + i
    sees every key at a position <= its own."""
    j = np.arange(n_kv)[None, :]
    i = q_pos0 + np.arange(n_q)[:, None]
    return np.where(j <= i, 0.0, NEG_INF)


def attention_rows(q, k_pool, v_pool, kv_rows, scale, mask=None, softcap=0.0):
    """Unified-pool attention.

    q (n_seq, n_head, n_q, d); k_pool/v_pool (n_head_kv, n_pool, d); kv_rows (n_seq, n_kv)
    int; mask (n_seq, n_q, n_kv) or None.  Returns O (n_seq, n_q, n_head, dv) and
    LSE (n_seq, n_q, n_head)."""
    n_seq = q.shape[0]
    outs, lses = [], []
    for b in range(n_seq):
        rows = np.asarray(kv_rows[b])
        keep = rows >= 0
        r = rows[keep].astype(np.int64)
        m = None if mask is None else np.asarray(mask[b], dtype=np.float64)[:, keep]
        O, L = attention(q[b], k_pool[:, r], v_pool[:, r], scale, m, softcap)
        outs.append(O)
        lses.append(L)
    return np.stack(outs), np.stack(lses)
