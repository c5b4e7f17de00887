"""rkv: split-KV (device window + pinned-host tail, or row-list pool) flash attention for
AMD Instinct MI355X.  Python binding of librkv.so; torch supplies device memory, pinned
host memory and streams, every step of the attention runs in the library's HIP kernels.

Tensor conventions (numpy/torch C order, last axis fastest; ggml shapes in brackets):
  * q       float16 (n_head, n_q, 128)            [128, n_q, n_head]
            rows variant: (n_seq, n_head, n_q, 128) [128, n_q, n_head, n_seq]
  * K / V   uint8 cell-major cache (n_cells, n_head_kv, row_bytes) or head-major
            (n_head_kv, n_cells, row_bytes); row_bytes 256 (f16), 136 (q8_0), 72 (q4_0)
  * mask    float16 (n_q, n_kv) additive; rows variant (n_seq, 1, n_q, n_kv)
  * o       float32 (n_q, n_head, 128); lse float32 (n_q, n_head)
"""
from __future__ import annotations

import ctypes

from ._lib import (RKV_LIFT_AUTO, RKV_LIFT_BULK, RKV_LIFT_DIRECT, RKV_LIFT_KERNEL, RKV_LIFT_UVA, RKV_RESIDENCY_AUTO, RKV_RESIDENCY_RESIDENT,  # noqa: F401
                   RKV_RESIDENCY_WINDOW, RKV_TAIL_HOST, RKV_DQ_DECODE_MMA, RKV_DQ_PREFILL, RKV_DQ_VECTOR, RKV_DQ_HEAD_DIM, RKV_TAIL_LIFT, RKV_TYPE_F16, RKV_TYPE_F32, RKV_TYPE_Q4_0,
                   RKV_TYPE_Q8_0, RKV_ERR_ARG, RKV_ERR_UNSUPPORTED, RkvError,
                   RkvBcacheCounters, RkvStats, RkvTensor, check, load)

BLOCK_BYTES = {RKV_TYPE_F16: 2, RKV_TYPE_F32: 4, RKV_TYPE_Q8_0: 34, RKV_TYPE_Q4_0: 18}
ROW_BYTES = {RKV_TYPE_F16: 256, RKV_TYPE_Q8_0: 136, RKV_TYPE_Q4_0: 72}


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def tensor(data_ptr: int, type_id: int, ne, nb) -> RkvTensor:
    t = RkvTensor()
    t.data = ctypes.c_void_p(int(data_ptr))
    t.type = int(type_id)
    for i in range(4):
        t.ne[i] = int(ne[i]) if i < len(ne) else 1
        t.nb[i] = int(nb[i]) if i < len(nb) else int(t.nb[i - 1] * t.ne[i - 1])
    return t


def q_desc(q) -> RkvTensor:
    """float16 q (n_head, n_q, 128) or (n_seq, n_head, n_q, 128)."""
    es = q.element_size()
    if q.dim() == 3:
        h, n, d = q.shape
        return tensor(q.data_ptr(), RKV_TYPE_F16, [d, n, h, 1],
                      [es, q.stride(1) * es, q.stride(0) * es, q.stride(0) * es * h])
    s, h, n, d = q.shape
    return tensor(q.data_ptr(), RKV_TYPE_F16, [d, n, h, s],
                  [es, q.stride(2) * es, q.stride(1) * es, q.stride(0) * es])


def kv_desc(cache, type_id: int, layout: str = "cell") -> RkvTensor:
    """uint8 cache: cell-major (n_cells, n_head_kv, row_bytes) or head-major
    (n_head_kv, n_cells, row_bytes) -> [d, n_cells, n_head_kv, 1], with the head dim d read
    off the row size (a row of 128 values is ROW_BYTES[type_id] bytes)."""
    if layout == "cell":
        n_cells, n_head_kv, row = cache.shape
        nb1, nb2 = cache.stride(0), cache.stride(1)
    else:
        n_head_kv, n_cells, row = cache.shape
        nb1, nb2 = cache.stride(1), cache.stride(0)
    assert (row * 128) % ROW_BYTES[type_id] == 0 and cache.stride(2) == 1, "rows must be contiguous whole rows"
    d = row * 128 // ROW_BYTES[type_id]
    return tensor(cache.data_ptr(), type_id, [d, n_cells, n_head_kv, 1],
                  [BLOCK_BYTES[type_id], nb1, nb2, nb2 * n_head_kv])


def mask_desc(mask) -> RkvTensor | None:
    """float16 mask (n_q, n_kv) or (n_seq, 1, n_q, n_kv)."""
    if mask is None:
        return None
    es = mask.element_size()
    if mask.dim() == 2:
        n_q, n_kv = mask.shape
        return tensor(mask.data_ptr(), RKV_TYPE_F16, [n_kv, n_q, 1, 1],
                      [es, mask.stride(0) * es, mask.stride(0) * es * n_q, mask.stride(0) * es * n_q])
    s, one, n_q, n_kv = mask.shape
    return tensor(mask.data_ptr(), RKV_TYPE_F16, [n_kv, n_q, one, s],
                  [es, mask.stride(2) * es, mask.stride(1) * es, mask.stride(0) * es])


def _ref(t):
    return None if t is None else ctypes.byref(t)


class Context:
    """Owns an rkv_ctx (copy stream, events, scratch ring, partials workspace)."""

    def __init__(self, device: int = 0):
        self.lib = load()
        h = ctypes.c_void_p()
        check(self.lib.rkv_create(int(device), ctypes.byref(h)), "rkv_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.rkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- configuration
    def reserve(self, max_tile_bytes_k=0, max_tile_bytes_v=0, n_slots=0, max_partial_floats=0):
        check(self.lib.rkv_reserve(self.h, int(max_tile_bytes_k), int(max_tile_bytes_v), int(n_slots),
                                   int(max_partial_floats)), "rkv_reserve")

    def set_lift_mode(self, mode: int):
        check(self.lib.rkv_set_lift_mode(self.h, int(mode)), "rkv_set_lift_mode")

    def set_direct_tail_max(self, nbytes: int):
        check(self.lib.rkv_set_direct_tail_max(self.h, int(nbytes)), "rkv_set_direct_tail_max")

    def set_splits(self, splits: int):
        check(self.lib.rkv_set_splits(self.h, int(splits)), "rkv_set_splits")

    def set_softcap(self, softcap: float):
        """Logit soft-cap of later calls: scale*qk -> softcap*tanh(scale*qk/softcap); 0 = off."""
        check(self.lib.rkv_set_softcap(self.h, float(softcap)), "rkv_set_softcap")

    def set_tail_mode(self, mode: int, n_threads: int = 0):
        """RKV_TAIL_LIFT (default) or RKV_TAIL_HOST: decode computes a host tail's partial on
        n_threads host threads (0 = all) while the GPU computes the window."""
        check(self.lib.rkv_set_tail_mode(self.h, int(mode), int(n_threads)), "rkv_set_tail_mode")

    def set_lift_timing(self, on: bool):
        check(self.lib.rkv_set_lift_timing(self.h, int(bool(on))), "rkv_set_lift_timing")

    def lift_timing_ms(self):
        tot, span, n = ctypes.c_float(), ctypes.c_float(), ctypes.c_int()
        check(self.lib.rkv_lift_timing_ms(self.h, ctypes.byref(tot), ctypes.byref(span), ctypes.byref(n)),
              "rkv_lift_timing_ms")
        return tot.value, span.value, n.value

    def set_kernel_timing(self, on: bool):
        check(self.lib.rkv_set_kernel_timing(self.h, int(bool(on))), "rkv_set_kernel_timing")

    def kernel_timing_ms(self):
        tot, n = ctypes.c_float(), ctypes.c_int()
        check(self.lib.rkv_kernel_timing_ms(self.h, ctypes.byref(tot), ctypes.byref(n)), "rkv_kernel_timing_ms")
        return tot.value, n.value

    def stats(self) -> dict:
        s = RkvStats()
        check(self.lib.rkv_get_stats(self.h, ctypes.byref(s)), "rkv_get_stats")
        return {f: getattr(s, f) for f, _ in RkvStats._fields_}

    # -- attention
    def attn_decode(self, q, k_win, v_win, k_tail, v_tail, mask, wc, tile_kv, scale, o, lse=None,
                    stream=None):
        """Tensors are rkv_tensor descriptors (see q_desc / kv_desc / mask_desc) or None."""
        check(self.lib.rkv_attn_decode(self.h, _ref(q), _ref(k_win), _ref(v_win), _ref(k_tail), _ref(v_tail),
                                       _ref(mask), int(wc), int(tile_kv), float(scale), _ptr(o), _ptr(lse),
                                       _stream(stream)), "rkv_attn_decode")

    def attn_prefill(self, q, k_win, v_win, k_tail, v_tail, mask, wc, tile_kv, scale, q_pos0, o, lse=None,
                     stream=None):
        check(self.lib.rkv_attn_prefill(self.h, _ref(q), _ref(k_win), _ref(v_win), _ref(k_tail), _ref(v_tail),
                                        _ref(mask), int(wc), int(tile_kv), float(scale), int(q_pos0), _ptr(o),
                                        _ptr(lse), _stream(stream)), "rkv_attn_prefill")

    def attn_rows(self, q, k_pool, v_pool, kv_rows, n_kv, mask, scale, o, lse=None, stream=None):
        check(self.lib.rkv_attn_rows(self.h, _ref(q), _ref(k_pool), _ref(v_pool), _ptr(kv_rows), int(n_kv),
                                     _ref(mask), float(scale), _ptr(o), _ptr(lse), _stream(stream)),
              "rkv_attn_rows")

    def attn_partial(self, q, k, v, mask, kv_pos0, q_pos0, scale, partial, stream=None):
        check(self.lib.rkv_attn_partial(self.h, _ref(q), _ref(k), _ref(v), _ref(mask), int(kv_pos0),
                                        int(q_pos0), float(scale), _ptr(partial), _stream(stream)),
              "rkv_attn_partial")

    def tail_lift(self, host_src, nbytes: int, slot: int, mode: int = RKV_LIFT_BULK, copy_stream=None) -> int:
        dst = ctypes.c_void_p()
        cs = ctypes.c_void_p(0) if copy_stream is None else _stream(copy_stream)
        check(self.lib.rkv_tail_lift(self.h, _ptr(host_src), int(nbytes), int(slot), int(mode),
                                     ctypes.byref(dst), cs), "rkv_tail_lift")
        return int(dst.value or 0)


class BlockCache:
    """Device-side block cache over a pinned host copy (rkv_bcache_*): k_host / v_host are pinned
    uint8 caches (n_cells, n_head_kv, row_bytes) the caller keeps alive."""

    def __init__(self, k_host, v_host, k_type: int, v_type: int, page_size: int, n_slots: int):
        self.lib = load()
        self.k_host, self.v_host = k_host, v_host
        h = ctypes.c_void_p()
        kd, vd = kv_desc(k_host, k_type), kv_desc(v_host, v_type)
        check(self.lib.rkv_bcache_create(ctypes.byref(kd), ctypes.byref(vd), int(page_size), int(n_slots),
                                         ctypes.byref(h)), "rkv_bcache_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.rkv_bcache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, stream=None):
        check(self.lib.rkv_bcache_reset(self.h, _stream(stream)), "rkv_bcache_reset")

    def resolve(self, sel, rows=None, stream=None):
        """sel: int32 device tensor (n_seq, n_sel) of cell ids (-1 padding); rows: int32 device
        tensor of the same shape receiving slot-pool rows, or None."""
        n_seq, n_sel = (1, sel.shape[0]) if sel.dim() == 1 else (sel.shape[0], sel.shape[1])
        check(self.lib.rkv_bcache_resolve(self.h, _ptr(sel), int(n_sel), int(n_seq), _ptr(rows), _stream(stream)),
              "rkv_bcache_resolve")

    def pools(self):
        k, v = RkvTensor(), RkvTensor()
        check(self.lib.rkv_bcache_pools(self.h, ctypes.byref(k), ctypes.byref(v)), "rkv_bcache_pools")
        return k, v

    def append(self, k_cell, v_cell, cell: int, stream=None):
        check(self.lib.rkv_bcache_append(self.h, _ptr(k_cell), _ptr(v_cell), int(cell), _stream(stream)),
              "rkv_bcache_append")

    def counters(self) -> dict:
        c = RkvBcacheCounters()
        check(self.lib.rkv_bcache_counters(self.h, ctypes.byref(c)), "rkv_bcache_counters")
        return {f: getattr(c, f) for f, _ in RkvBcacheCounters._fields_}

    def map_arrays(self):
        """(page_table, slot_page) copied to host numpy arrays (synchronises the device)."""
        import numpy as np
        import torch
        pt, sp = ctypes.c_void_p(), ctypes.c_void_p()
        n_pages, n_slots = ctypes.c_int64(), ctypes.c_int64()
        check(self.lib.rkv_bcache_map(self.h, ctypes.byref(pt), ctypes.byref(sp), ctypes.byref(n_pages),
                                      ctypes.byref(n_slots)), "rkv_bcache_map")
        torch.cuda.synchronize()
        a = np.empty(n_pages.value, dtype=np.int32)
        b = np.empty(n_slots.value, dtype=np.int32)
        lib_hip = _hip()
        lib_hip.hipMemcpy.restype = ctypes.c_int
        lib_hip.hipMemcpy(ctypes.c_void_p(a.ctypes.data), pt, ctypes.c_size_t(a.nbytes), 2)
        lib_hip.hipMemcpy(ctypes.c_void_p(b.ctypes.data), sp, ctypes.c_size_t(b.nbytes), 2)
        return a, b


def _hip():
    """The HIP runtime the process already uses (the one torch loaded)."""
    import torch  # noqa: F401
    return ctypes.CDLL("libamdhip64.so")


def attn_decode_noalloc(q, k, v, mask, scale, o, lse=None, stream=None):
    """rkv_attn_decode over a device-resident cache with no context and no allocation: the
    partials live in the library's static device array (calls on one GPU must not overlap)."""
    lib = load()
    check(lib.rkv_attn_decode_noalloc(_ref(q), _ref(k), _ref(v), _ref(mask), float(scale), _ptr(o), _ptr(lse),
                                      _stream(stream)), "rkv_attn_decode_noalloc")


def lse_merge(partials, n_seg: int, n_rows: int, o, lse=None, stream=None, dv: int = 128):
    lib = load()
    check(lib.rkv_lse_merge(_ptr(partials), int(n_seg), int(n_rows), int(dv), _ptr(o), _ptr(lse), _stream(stream)),
          "rkv_lse_merge")


def tail_partial_host(q, k, v, mask, kv_pos0: int, q_pos0: int, scale: float, partial, softcap: float = 0.0,
                      n_threads: int = 0):
    """Tail partial on the host cores: q, k, v, mask are descriptors of host (CPU) memory,
    partial a float32 CPU tensor (n_q, n_head, 2 + dv) receiving (M, S, VKQ) per row."""
    lib = load()
    check(lib.rkv_tail_partial_host(_ref(q), _ref(k), _ref(v), _ref(mask), int(kv_pos0), int(q_pos0),
                                    float(scale), float(softcap), _ptr(partial), int(n_threads)),
          "rkv_tail_partial_host")


def choose_tail_mode(tail_bytes: int, h2d_gbps: float, host_gbps: float) -> int:
    """RKV_TAIL_HOST when the host cores read the tail faster than the link lifts it, else RKV_TAIL_LIFT."""
    lib = load()
    m = ctypes.c_int()
    check(lib.rkv_choose_tail_mode(int(tail_bytes), float(h2d_gbps), float(host_gbps), ctypes.byref(m)),
          "rkv_choose_tail_mode")
    return m.value


def dequant_rows(src, type_id: int, n_rows: int, row_stride: int, dst, stream=None, form: int = RKV_DQ_DECODE_MMA,
                 row_values: int = 128):
    """Rows of row_values values rebuilt through the unpack routines of kernel family `form`."""
    lib = load()
    check(lib.rkv_dequant_rows(_ptr(src), int(type_id), int(form), int(n_rows), int(row_values), int(row_stride),
                               _ptr(dst), _stream(stream)), "rkv_dequant_rows")


def plan_window(per_cell: int, kv_size: int, free_bytes: int = -1, target_bytes: int = 0,
                reserve_bytes: int = 3 << 29, align: int = 256, ctx: "Context | None" = None) -> int:
    """Resident cells of a position-windowed cache (rkv_plan_window); free_bytes < 0 reads the
    free memory of ctx's device.  The default reserve is 1.5 GiB."""
    lib = load()
    wc = ctypes.c_int64()
    check(lib.rkv_plan_window(ctx.h if ctx is not None else None, int(per_cell), int(kv_size), int(free_bytes),
                              int(target_bytes), int(reserve_bytes), int(align), ctypes.byref(wc)),
          "rkv_plan_window")
    return int(wc.value)


def window_mode(mode: int, wc: int, kv_size: int, append_only: bool = True, v_transposed: bool = False) -> bool:
    """Whether the cache runs as window + tail (rkv_window_mode)."""
    lib = load()
    out = ctypes.c_int()
    check(lib.rkv_window_mode(int(mode), int(wc), int(kv_size), int(bool(append_only)), int(bool(v_transposed)),
                              ctypes.byref(out)), "rkv_window_mode")
    return bool(out.value)


def version() -> str:
    return load().rkv_version().decode()
