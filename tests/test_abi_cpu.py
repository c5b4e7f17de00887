"""Host-side checks of the C ABI that need no GPU: the library loads, exports every symbol
include/rkv.h declares (and the Python binding declares the same set), and argument
errors are reported as status codes before any device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from tiered_kv_cache_split_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("librkv.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("rkv_attn_decode", "rkv_attn_prefill", "rkv_attn_rows", "rkv_lse_merge",
                     "rkv_tail_lift"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_binding_matches_header():
    from tiered_kv_cache_split_amd import _lib
    assert sorted(_lib.SIGNATURES) == header_functions()


def test_version_and_strerror(lib):
    assert re.match(r"^\d+\.\d+\.\d+$", lib.rkv_version().decode())
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.rkv_strerror(st).decode() not in ("", "unknown status")
    assert lib.rkv_strerror(42).decode() == "unknown status"


def test_null_context_is_an_argument_error(lib):
    from tiered_kv_cache_split_amd import _lib
    assert lib.rkv_attn_decode(None, None, None, None, None, None, None, 0, 1, 1.0, None, None, None) == _lib.RKV_ERR_ARG
    assert lib.rkv_attn_rows(None, None, None, None, None, 0, None, 1.0, None, None, None) == _lib.RKV_ERR_ARG
    assert lib.rkv_attn_prefill(None, None, None, None, None, None, None, 0, 1, 1.0, -1, None, None, None) == _lib.RKV_ERR_ARG
    assert lib.rkv_reserve(None, 0, 0, 2, 0) == _lib.RKV_ERR_ARG
    assert lib.rkv_set_direct_tail_max(None, 0) == _lib.RKV_ERR_ARG
    assert b"ctx" in lib.rkv_last_error()
    d = ctypes.c_void_p()
    assert lib.rkv_tail_lift(None, None, 0, 0, 0, ctypes.byref(d), None) == _lib.RKV_ERR_ARG
    lib.rkv_destroy(None)  # no-op


def test_merge_rejects_bad_sizes_before_device_work(lib):
    from tiered_kv_cache_split_amd import _lib
    for dv in (32, 96, 576, 1024):  # value widths other than 64, 128, 256 and 512
        assert lib.rkv_lse_merge(None, 2, 4, dv, None, None, None) == _lib.RKV_ERR_UNSUPPORTED
    assert lib.rkv_lse_merge(None, 0, 4, 512, None, None, None) == _lib.RKV_ERR_ARG  # 512 passes the width check
    assert lib.rkv_lse_merge(None, 0, 4, 64, None, None, None) == _lib.RKV_ERR_ARG
    assert lib.rkv_lse_merge(None, 0, 4, 128, None, None, None) == _lib.RKV_ERR_ARG
    assert lib.rkv_lse_merge(None, 1, 0, 128, None, None, None) == _lib.RKV_OK  # nothing to do


def test_dequant_rejects_unknown_type(lib):
    from tiered_kv_cache_split_amd import _lib
    assert lib.rkv_dequant_rows(None, 3, 0, 4, 128, 256, None, None) == _lib.RKV_ERR_UNSUPPORTED
    assert lib.rkv_dequant_rows(None, 8, 0, 4, 128, 100, None, None) == _lib.RKV_ERR_ARG  # row_stride < 136
    assert lib.rkv_dequant_rows(None, 8, 4, 4, 128, 136, None, None) == _lib.RKV_ERR_ARG  # unknown form
    assert lib.rkv_dequant_rows(None, 8, 0, 4, 100, 136, None, None) == _lib.RKV_ERR_ARG  # row_values % 32
    assert lib.rkv_dequant_rows(None, 8, 0, 0, 128, 136, None, None) == _lib.RKV_OK      # nothing to do


def test_descriptor_layouts():
    """The binding's descriptors follow the ggml convention (ne[0] fastest, byte strides)."""
    torch = pytest.importorskip("torch")
    import tiered_kv_cache_split_amd as rkv
    q = torch.zeros(40, 3, 128, dtype=torch.float16)
    d = rkv.q_desc(q)
    assert list(d.ne) == [128, 3, 40, 1] and list(d.nb)[:3] == [2, 256, 3 * 256]
    k = torch.zeros(100, 8, 136, dtype=torch.uint8)
    d = rkv.kv_desc(k, rkv.RKV_TYPE_Q8_0, "cell")
    assert list(d.ne) == [128, 100, 8, 1] and list(d.nb)[:3] == [34, 8 * 136, 136]
    kh = torch.zeros(8, 100, 72, dtype=torch.uint8)
    d = rkv.kv_desc(kh, rkv.RKV_TYPE_Q4_0, "head")
    assert list(d.ne) == [128, 100, 8, 1] and list(d.nb)[:3] == [18, 72, 100 * 72]
    for d_, t, rb in [(64, rkv.RKV_TYPE_Q8_0, 68), (256, rkv.RKV_TYPE_Q4_0, 144), (64, rkv.RKV_TYPE_F16, 128)]:
        d = rkv.kv_desc(torch.zeros(10, 2, rb, dtype=torch.uint8), t)  # head dim read off the row size
        assert list(d.ne) == [d_, 10, 2, 1] and list(d.nb)[:3] == [rkv.BLOCK_BYTES[t], 2 * rb, rb]
    m = torch.zeros(3, 500, dtype=torch.float16)
    d = rkv.mask_desc(m)
    assert list(d.ne) == [500, 3, 1, 1] and list(d.nb)[:2] == [2, 1000]


def test_no_device_is_reported(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from tiered_kv_cache_split_amd import _lib
    h = ctypes.c_void_p()
    assert lib.rkv_create(0, ctypes.byref(h)) == _lib.RKV_ERR_HIP


# ---- residency policy: host arithmetic, checked against the oracle without a GPU

def test_plan_window_matches_the_oracle(lib):
    import numpy as np
    import oracle
    import tiered_kv_cache_split_amd as rkv
    rng = np.random.default_rng(77)
    cases = [(1664, 262144, 300 << 30, 0, 3 << 29, 256), (79872, 1 << 20, 300 << 30, 64 << 30, 3 << 29, 256),
             (512, 0, 1 << 30, 0, 0, 32), (1, 1, 0, 0, 0, 1), (1 << 40, 1 << 20, 1 << 62, 0, 0, 1 << 20)]
    for _ in range(3000):
        per_cell = int(rng.integers(1, 1 << 20))
        kv = int(rng.integers(0, 1 << 22))
        free = int(rng.integers(0, 1 << 45))
        target = int(rng.choice([0, int(rng.integers(1, 1 << 45))]))
        reserve = int(rng.integers(0, 1 << 33))
        align = int(rng.choice([1, 32, 256, 1024]))
        cases.append((per_cell, kv, free, target, reserve, align))
    for c in cases:
        assert rkv.plan_window(*c) == oracle.plan_window(*c), c


def test_plan_window_argument_errors(lib):
    from tiered_kv_cache_split_amd import _lib
    wc = ctypes.c_int64()
    for args in [(0, 10, 100, 0, 0, 32), (16, -1, 100, 0, 0, 32), (16, 10, 100, 0, 0, 0), (16, 10, 100, 0, -1, 32),
                 (16, 10, -1, 0, 0, 32)]:  # the last: free < 0 needs a context
        assert lib.rkv_plan_window(None, *args, ctypes.byref(wc)) == _lib.RKV_ERR_ARG, args
    assert lib.rkv_plan_window(None, 16, 10, 100, 0, 0, 32, None) == _lib.RKV_ERR_ARG


def test_window_mode_matches_the_oracle(lib):
    import oracle
    import tiered_kv_cache_split_amd as rkv
    from tiered_kv_cache_split_amd import _lib
    for mode in (0, 1, 2):
        for wc in (0, 1, 500, 999, 1000, 1001):
            for ao in (False, True):
                for vt in (False, True):
                    assert rkv.window_mode(mode, wc, 1000, ao, vt) == oracle.window_mode(mode, wc, 1000, ao, vt)
    out = ctypes.c_int()
    assert lib.rkv_window_mode(3, 1, 2, 1, 0, ctypes.byref(out)) == _lib.RKV_ERR_ARG
    assert lib.rkv_window_mode(0, 1, 2, 1, 0, None) == _lib.RKV_ERR_ARG
