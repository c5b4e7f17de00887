"""Pins for the fp64 oracle against facts fixed by the pages and by the mathematics.

None of these re-types the oracle's formula: each compares it with something
independent -- pure-Python brute force, closed forms, a library routine on a
special case, hand-made format fixtures, or an algebraic invariant of the
segment split.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import quant as oq
import rkv_inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG = -math.inf


# ------------------------------------------------------------- brute force
def brute_attention(q, k, v, scale, mask):
    """Pure-Python loops with math.fsum/math.exp; q (H,Q,d), k/v (G,N,d), mask (Q,N) or None."""
    H, Qn, d = q.shape
    G, N, dv = v.shape
    gqa = H // G
    O = np.zeros((Qn, H, dv))
    L = np.full((Qn, H), NEG)
    for i in range(Qn):
        for h in range(H):
            g = h // gqa
            s = []
            for j in range(N):
                x = scale * math.fsum(float(q[h, i, t]) * float(k[g, j, t]) for t in range(d))
                if mask is not None:
                    x += float(mask[i, j])
                s.append(x)
            vis = [j for j in range(N) if s[j] != NEG]
            if not vis:
                continue
            m = max(s[j] for j in vis)
            tot = math.fsum(math.exp(s[j] - m) for j in vis)
            lse = m + math.log(tot)
            L[i, h] = lse
            for t in range(dv):
                O[i, h, t] = math.fsum(math.exp(s[j] - lse) * float(v[g, j, t]) for j in vis)
    return O, L


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    H, G, Qn, N, d = 6, 2, 3, 11, 8
    q = rng.standard_normal((H, Qn, d))
    k = rng.standard_normal((G, N, d))
    v = rng.standard_normal((G, N, d))
    mask = np.where(rng.random((Qn, N)) < 0.3, NEG, rng.standard_normal((Qn, N)))
    mask[2, :] = NEG  # one fully hidden query row
    O, L = oracle.attention(q, k, v, 0.37, mask)
    Ob, Lb = brute_attention(q, k, v, 0.37, mask)
    assert np.allclose(O, Ob, atol=1e-13, rtol=0)
    fin = np.isfinite(Lb)
    assert np.array_equal(np.isfinite(L), fin)
    assert np.allclose(L[fin], Lb[fin], atol=1e-13, rtol=0)
    assert np.all(O[2] == 0.0) and np.all(L[2] == NEG)


# ------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(5)
    G, N, d = 2, 9, 8
    q = np.zeros((4, 1, d))
    k = rng.standard_normal((G, N, d))
    v = rng.standard_normal((G, N, d))
    mask = np.zeros((1, N))
    mask[0, [1, 4]] = NEG
    keep = [j for j in range(N) if j not in (1, 4)]
    O, L = oracle.attention(q, k, v, 1.0, mask)
    for h in range(4):
        assert np.allclose(O[0, h], v[h // 2, keep].mean(axis=0), atol=1e-14)
        assert abs(L[0, h] - math.log(len(keep))) < 1e-14


def test_single_visible_key():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 1, 8))
    k = rng.standard_normal((1, 5, 8))
    v = rng.standard_normal((1, 5, 8))
    mask = np.full((1, 5), NEG)
    mask[0, 3] = 0.25
    O, L = oracle.attention(q, k, v, 0.5, mask)
    for h in range(2):
        assert np.allclose(O[0, h], v[0, 3], atol=1e-15)
        assert abs(L[0, h] - (0.5 * float(q[h, 0] @ k[0, 3]) + 0.25)) < 1e-14


def test_two_keys_sigmoid_weights():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    s0, s1 = [0.7 * float(q[0, 0] @ k[0, j]) for j in range(2)]
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    O, L = oracle.attention(q, k, v, 0.7, None)
    assert np.allclose(O[0, 0], (1 - w1) * v[0, 0] + w1 * v[0, 1], atol=1e-14)
    assert abs(L[0, 0] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-13


def test_logit_shift_and_value_scaling():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 2, 8))
    k = rng.standard_normal((2, 10, 8))
    v = rng.standard_normal((2, 10, 8))
    O, L = oracle.attention(q, k, v, 0.3, None)
    O2, L2 = oracle.attention(q, k, v, 0.3, np.full((2, 10), 1.75))
    assert np.allclose(O2, O, atol=1e-14) and np.allclose(L2, L + 1.75, atol=1e-13)
    O3, L3 = oracle.attention(q, k, 3.0 * v, 0.3, None)
    assert np.allclose(O3, 3.0 * O, atol=1e-13) and np.allclose(L3, L, atol=0)


@pytest.mark.parametrize("d", [16, 64, 256])
def test_library_special_case_sdpa_f64(d):
    """torch SDPA on CPU in float64 with the KV heads repeated for the grouped-query map."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    H, G, Qn, N = 8, 2, 5, 37
    q = rng.standard_normal((H, Qn, d))
    k = rng.standard_normal((G, N, d))
    v = rng.standard_normal((G, N, d))
    mask = np.where(rng.random((Qn, N)) < 0.2, NEG, 0.3 * rng.standard_normal((Qn, N)))
    O, _ = oracle.attention(q, k, v, 0.21, mask)
    kr = torch.from_numpy(k).repeat_interleave(H // G, dim=0)
    vr = torch.from_numpy(v).repeat_interleave(H // G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], kr[None], vr[None], attn_mask=torch.from_numpy(mask), scale=0.21)
    ref = ref[0].permute(1, 0, 2).numpy()  # (Q, H, d)
    assert np.allclose(O, ref, atol=1e-12)


def test_library_special_case_sdpa_f64_dk_ne_dv():
    """dk = 576, dv = 512 (Q/K wider than V): torch SDPA in float64 takes the two widths too."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(19)
    H, G, Qn, N, dk, dv = 8, 1, 2, 29, 576, 512
    q = rng.standard_normal((H, Qn, dk))
    k = rng.standard_normal((G, N, dk))
    v = rng.standard_normal((G, N, dv))
    mask = np.where(rng.random((Qn, N)) < 0.2, NEG, 0.3 * rng.standard_normal((Qn, N)))
    O, L = oracle.attention(q, k, v, 0.04, mask)
    assert O.shape == (Qn, H, dv) and L.shape == (Qn, H)
    kr = torch.from_numpy(k).repeat_interleave(H // G, dim=0)
    vr = torch.from_numpy(v).repeat_interleave(H // G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], kr[None], vr[None], attn_mask=torch.from_numpy(mask), scale=0.04)
    assert np.allclose(O, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)
    # LSE against its definition with math.fsum on one row
    s = [0.04 * math.fsum(q[3, 1] * k[0, j]) + mask[1, j] for j in range(N)]
    m = max(x for x in s if x > -np.inf)
    assert abs(L[1, 3] - (m + math.log(math.fsum(math.exp(x - m) for x in s if x > -np.inf)))) < 1e-12


# ------------------------------------------------------------- split method
@pytest.mark.parametrize("seed", range(4))
def test_partition_invariance(seed):
    rng = np.random.default_rng(100 + seed)
    H, G, Qn, N, d = 10, 2, 3, 97, 16
    q = rng.standard_normal((H, Qn, d))
    k = rng.standard_normal((G, N, d)) * (1 + 4 * (rng.random((G, N, 1)) < 0.1))
    v = rng.standard_normal((G, N, d))
    mask = np.where(rng.random((Qn, N)) < 0.25, NEG, 0.0)
    inner = sorted(rng.integers(0, N + 1, size=int(rng.integers(1, 9))).tolist())
    cuts = [0] + inner + [inner[-1], N]  # repeated cut = an empty segment, a no-op
    O, L = oracle.attention(q, k, v, 0.25, mask)
    Os, Ls = oracle.split_attention(q, k, v, 0.25, mask, cuts)
    assert np.allclose(Os, O, atol=1e-13)
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(Ls), fin) and np.allclose(Ls[fin], L[fin], atol=1e-13)


def test_empty_tail_is_single_resident():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 1, 8))
    k = rng.standard_normal((1, 40, 8))
    v = rng.standard_normal((1, 40, 8))
    b = oracle.window_tail_bounds(40, 40, 16)
    assert b == [0, 40]
    O, L = oracle.split_attention(q, k, v, 0.5, None, b)
    O1, L1 = oracle.attention(q, k, v, 0.5, None)
    assert np.array_equal(O, O1) and np.array_equal(L, L1)


def test_window_tail_tiling_never_straddles():
    assert oracle.window_tail_bounds(4096, 2048, 1024) == [0, 2048, 3072, 4096]
    assert oracle.window_tail_bounds(106496, 65536, 32768) == [0, 65536, 98304, 106496]
    assert oracle.window_tail_bounds(262144, 131072, 32768) == [0, 131072] + [131072 + 32768 * t
                                                                            for t in range(1, 5)]
    assert oracle.window_tail_bounds(100, 0, 31) == [0, 31, 62, 93, 100]
    b = oracle.window_tail_bounds(1000, 333, 256)
    assert 333 in b and b[-1] == 1000 and all(y - x <= 256 for x, y in zip(b[1:], b[2:]))


def test_partial_roundtrip_no_double_count():
    """O = VKQ/S and LSE = M + ln S for a single partial (patch 0070 tail-partial rule)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 1, 8))
    k = rng.standard_normal((1, 30, 8))
    v = rng.standard_normal((1, 30, 8))
    M, S, VKQ = oracle.partial(q, k, v, 0.4, None)
    O, L = oracle.attention(q, k, v, 0.4, None)
    assert np.allclose(VKQ / S[..., None], O, atol=1e-14)
    assert np.allclose(M + np.log(S), L, atol=1e-14)
    Ob, Lb = brute_attention(q, k, v, 0.4, None)
    assert np.allclose(O, Ob, atol=1e-13)


def test_merge_empty_and_all_empty():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 1, 8))
    k = rng.standard_normal((1, 6, 8))
    v = rng.standard_normal((1, 6, 8))
    p = oracle.partial(q, k, v, 0.4, None)
    e = oracle.partial(q, k[:, :0], v[:, :0], 0.4, None)
    assert np.all(e[0] == NEG) and np.all(e[1] == 0)
    O, L = oracle.merge([e, p, e])
    O1, L1 = oracle.merge([p])
    assert np.array_equal(O, O1) and np.array_equal(L, L1)
    O2, L2 = oracle.merge([e, e])
    assert np.all(O2 == 0) and np.all(L2 == NEG)


def test_outlier_keys_against_brute_force():
    """Every 17th key scaled by 30 (the Strata streaming test's outlier pattern)."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 2, 8))
    k = rng.standard_normal((1, 60, 8))
    k[:, ::17] *= 30
    v = rng.standard_normal((1, 60, 8))
    O, L = oracle.attention(q, k, v, 1 / math.sqrt(8), None)
    Ob, Lb = brute_attention(q, k, v, 1 / math.sqrt(8), None)
    assert np.allclose(O, Ob, atol=1e-12) and np.allclose(L, Lb, atol=1e-12)


# ------------------------------------------------------------- rows / padding
def test_rows_padding_contributes_nothing():
    rng = np.random.default_rng(15)
    G, P, d = 2, 50, 8
    kp = rng.standard_normal((G, P, d))
    vp = rng.standard_normal((G, P, d))
    q = rng.standard_normal((2, 4, 1, d))
    rows = np.array([[3, 7, 9, 40, -1, -1], [0, 1, 2, 3, 4, 5]], dtype=np.int32)
    mask = np.zeros((2, 1, 6))
    mask[0, 0, 4:] = NEG
    O, L = oracle.attention_rows(q, kp, vp, rows, 0.3, mask)
    O0, L0 = oracle.attention(q[0], kp[:, [3, 7, 9, 40]], vp[:, [3, 7, 9, 40]], 0.3, None)
    assert np.allclose(O[0], O0, atol=1e-15) and np.allclose(L[0], L0, atol=1e-15)
    # a negative row contributes nothing whatever the mask says
    O2, L2 = oracle.attention_rows(q, kp, vp, rows, 0.3, np.zeros((2, 1, 6)))
    assert np.allclose(O2, O, atol=1e-15)
    # brute force through explicit gathering
    Ob, Lb = brute_attention(q[1], kp[:, :6], vp[:, :6], 0.3, None)
    assert np.allclose(O[1], Ob, atol=1e-13)


def test_rows_fully_padded_sequence():
    rng = np.random.default_rng(16)
    kp = rng.standard_normal((1, 10, 8))
    q = rng.standard_normal((1, 2, 1, 8))
    O, L = oracle.attention_rows(q, kp, kp, np.full((1, 4), -1, np.int32), 0.3, None)
    assert np.all(O == 0) and np.all(L == NEG)


def test_causal_mask_matches_positions():
    m = oracle.causal_mask(3, 6, 3)
    assert (m[0] == [0, 0, 0, 0, NEG, NEG]).all()
    assert (m[2] == 0).all()


# ------------------------------------------------------------- formats
def _read_golden(name):
    blocks, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(" ", 1)
            cur[key] = rest
            if key == "values":
                blocks.append(cur)
                cur = {}
    return blocks


def test_q8_0_golden_blocks():
    blocks = _read_golden("q8_0_blocks.txt")
    assert len(blocks) >= 5
    for b in blocks:
        raw = np.frombuffer(bytes.fromhex(b["bytes"]), dtype=np.uint8)
        want = np.array([float(x) for x in b["values"].split()])
        got = oq.decode_q8_0(raw[None])[0]
        assert np.array_equal(got, want), b["scale_bits"]


def test_q4_0_golden_blocks():
    blocks = _read_golden("q4_0_blocks.txt")
    assert len(blocks) >= 4
    for b in blocks:
        raw = np.frombuffer(bytes.fromhex(b["bytes"]), dtype=np.uint8)
        want = np.array([float(x) for x in b["values"].split()])
        got = oq.decode_q4_0(raw[None])[0]
        assert np.array_equal(got, want), b["scale_bits"]


def test_f16_decode_special_values():
    bits = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xC000, 0x7BFF], np.uint16)
    want = [0.0, -0.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 1.0, -2.0, 65504.0]
    got = oq.decode_f16(bits.view(np.uint8)[None])[0]
    assert np.array_equal(got, np.array(want)) and math.copysign(1, got[1]) < 0


@pytest.mark.parametrize("t", [gen.TYPE_Q8_0, gen.TYPE_Q4_0])
def test_quantise_then_decode_error_bound(t):
    """Generator bytes read back by the oracle lie within the quantiser's step of the draws."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    vals = oq.decode(t, gen.pack(t, x))
    blk = np.abs(x.reshape(-1, 32)).max(axis=1)
    step = blk / (127.0 if t == gen.TYPE_Q8_0 else 8.0)
    err = np.abs(vals - x).reshape(-1, 32).max(axis=1)
    # q8_0: half a step plus 127 codes times the binary16 rounding of d (2^-11 relative);
    # q4_0: a full step, since the code opposite the extreme clamps from 16 to 15.
    factor = 0.5 + 127 * 2.0 ** -11 if t == gen.TYPE_Q8_0 else 1.0 + 8 * 2.0 ** -11
    assert np.all(err <= step * factor + 1e-7)


def test_kv_values_cell_major_layout():
    """Cell-major caches (cell, head, row) map to (head, cell, d)."""
    raw = np.arange(2 * 3 * 4, dtype=np.float32).reshape(3, 2, 4).astype(np.float16)
    vals = oracle.kv_values(gen.TYPE_F16, raw.view(np.uint8))
    assert vals.shape == (2, 3, 4)
    assert vals[1, 2, 3] == float(raw[2, 1, 3])


# ---- residency sizer (patch 0070, KV-cache hunk: position-window sizing and mode rule)

GIB = 1 << 30


def test_plan_window_fits_exactly_or_not():
    # whole cache exactly at the budget: resident; one byte less: a tail appears
    per_cell, kv = 1664, 262144
    need = per_cell * kv
    assert oracle.plan_window(per_cell, kv, need + GIB, 0, GIB, 256) == kv
    wc = oracle.plan_window(per_cell, kv, need + GIB - 1, 0, GIB, 256)
    assert wc == kv - 256  # the largest aligned window that leaves a tail


def test_plan_window_closed_forms():
    # budget 100 cells' worth (after target cap and reserve) -> 96 at alignment 32
    per_cell = 1000
    assert oracle.plan_window(per_cell, 10_000, 10**12, 100_500 + 7, 7, 32) == 96
    # the target caps the free bytes; the reserve eats the rest -> one unit
    assert oracle.plan_window(per_cell, 10_000, 10**12, 5_000, 10**9, 32) == 32
    # zero budget -> one unit of window
    assert oracle.plan_window(per_cell, 10_000, 0, 0, 0, 256) == 256
    # cache shorter than one unit that does not fit stays resident
    assert oracle.plan_window(per_cell, 100, 0, 0, 0, 256) == 100
    assert oracle.plan_window(per_cell, 0, 0, 0, 0, 256) == 0


@pytest.mark.parametrize("seed", range(6))
def test_plan_window_is_the_largest_aligned_fit(seed):
    """Against the definition by enumeration: among aligned windows that fit the budget and
    leave at least one unit of tail, the largest (one unit when none fits)."""
    rng = np.random.default_rng(seed)
    for _ in range(200):
        per_cell = int(rng.integers(1, 5000))
        align = int(rng.choice([1, 16, 32, 256]))
        kv = int(rng.integers(1, 40)) * int(rng.choice([1, align])) + int(rng.integers(0, 3))
        free = int(rng.integers(0, per_cell * kv * 2 + 10))
        target = int(rng.choice([0, int(rng.integers(1, per_cell * kv * 2 + 10))]))
        reserve = int(rng.integers(0, per_cell * 5 + 1))
        wc = oracle.plan_window(per_cell, kv, free, target, reserve, align)
        budget = max(0, (min(free, target) if target > 0 else free) - reserve)
        if per_cell * kv <= budget:
            assert wc == kv
            continue
        fitting = [m for m in range(align, kv, align) if m * per_cell <= budget and kv - m >= align]
        tail_ok = [m for m in range(align, kv, align) if kv - m >= align]
        if fitting:
            expect = max(fitting)
        elif tail_ok or kv <= align:
            expect = align
        else:
            expect = align
        assert wc == min(expect, kv), (per_cell, kv, free, target, reserve, align, wc, expect)


def test_window_mode_rule():
    kv = 1000
    for mode in (0, 2):
        assert oracle.window_mode(mode, 500, kv, True, False)
        assert not oracle.window_mode(mode, kv, kv, True, False)   # no overflow
        assert not oracle.window_mode(mode, 0, kv, True, False)
        assert not oracle.window_mode(mode, 500, kv, False, False)  # rotating cells
        assert not oracle.window_mode(mode, 500, kv, True, True)    # transposed V
    assert not oracle.window_mode(1, 500, kv, True, False)


# ---- logit soft-cap (patch 0070, streaming_lse_kernel soft-cap branch: c*tanh(scale*qk/c) before the mask)

def test_softcap_brute_force_tiny():
    rng = np.random.default_rng(123)
    q = rng.standard_normal((2, 1, 4))
    k = rng.standard_normal((1, 5, 4)) * 4.0
    v = rng.standard_normal((1, 5, 3))
    mask = np.array([[0.0, -np.inf, 0.5, 0.0, -1.0]])
    c, scale = 2.5, 0.7
    O, L = oracle.attention(q, k, v, scale, mask, softcap=c)
    for h in range(2):
        s = []
        for j in range(5):
            raw = scale * math.fsum(q[h, 0, d] * k[0, j, d] for d in range(4))
            s.append(c * math.tanh(raw / c) + mask[0, j])
        vis = [j for j in range(5) if s[j] > -math.inf]
        lse = math.log(math.fsum(math.exp(s[j]) for j in vis))
        assert abs(L[0, h] - lse) < 1e-12
        for e in range(3):
            ref = math.fsum(math.exp(s[j] - lse) * v[0, j, e] for j in vis)
            assert abs(O[0, h, e] - ref) < 1e-12


def test_softcap_limits():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((4, 2, 128))
    k = rng.standard_normal((2, 50, 128))
    v = rng.standard_normal((2, 50, 128))
    # a huge cap is the plain score; every capped score lies in [-c, c]
    O0, L0 = oracle.attention(q, k, v, 0.09)
    O1, L1 = oracle.attention(q, k, v, 0.09, softcap=1e9)
    assert np.abs(O0 - O1).max() < 1e-12 and np.abs(L0 - L1).max() < 1e-12
    s = oracle.scores(q, k * 50.0, 0.09, softcap=3.0)
    assert np.all(np.abs(s) <= 3.0) and np.abs(s).max() > 2.9  # saturates at the cap
    # partition invariance holds with the cap too
    parts = [oracle.partial(q, k[:, a:b], v[:, a:b], 0.09, None, 3.0) for a, b in [(0, 7), (7, 7), (7, 50)]]
    Om, Lm = oracle.merge(parts)
    Oa, La = oracle.attention(q, k, v, 0.09, softcap=3.0)
    assert np.abs(Om - Oa).max() < 1e-12 and np.abs(Lm - La).max() < 1e-12


# ---- block cache residency policy (oracle/block_cache.py), pinned by hand-worked CLOCK runs
# and invariants of the policy statement (Strata, "KV streaming for the QSA layers")

def test_clock_cold_start_hand_order():
    """4 slots of 2 cells: cells 0,1,2,3,8 name pages 0, 1, 4 -> three misses into the free
    slots 0, 1, 2 in hand order; the hand stops at 3; lookups: one per run of equal pages."""
    c = oracle.ClockCache(n_pages=8, n_slots=4, page_size=2)
    victims, missed, ovf = c.resolve([[0, 1, 2, 3, 8]])
    assert victims == [0, 1, 2] and missed == [0, 1, 4] and not ovf
    assert c.hand == 3 and c.page_table[:5] == [0, 1, -1, -1, 2] and c.slot_page == [0, 1, 4, -1]
    assert (c.misses, c.lookups, c.calls) == (3, 3, 1)


def test_clock_second_chance():
    """After the cold start, pages 1 (hit), 5, 6: slot 3 is free and taken; slot 0 (page 0,
    referenced) loses its bit; slot 1 is used by this call and skipped; slot 2 (page 4,
    referenced) loses its bit; slot 3 is now this call's; slot 0, unreferenced, is taken.  The
    hand stops past slot 0; page 0 is evicted; page 4 stays with its bit cleared."""
    c = oracle.ClockCache(n_pages=8, n_slots=4, page_size=2)
    c.resolve([[0, 1, 2, 3, 8]])
    victims, missed, ovf = c.resolve([[2, 10, 12]])
    assert victims == [3, 0] and missed == [5, 6] and not ovf
    assert c.hand == 1
    assert c.page_table[0] == -1 and c.page_table[1] == 1 and c.page_table[4] == 2
    assert c.page_table[5] == 3 and c.page_table[6] == 0
    assert c.slot_ref == [1, 1, 0, 1]
    assert (c.misses, c.lookups, c.calls) == (5, 6, 2)


def test_clock_overflow_and_padding():
    c = oracle.ClockCache(n_pages=16, n_slots=2, page_size=4)
    victims, missed, ovf = c.resolve([[0, 4, -1, 8, -1, -1]])
    assert ovf and len(victims) == 2 and len(missed) == 2 and c.overflow
    assert c.lookups == 3  # padding never counts


def test_clock_invariants_random():
    """Random calls: the map is its own inverse, every page a call names is resident after it,
    residency never exceeds the slots, and the victims are distinct slots."""
    rng = np.random.default_rng(8)
    c = oracle.ClockCache(n_pages=64, n_slots=12, page_size=4)
    for _ in range(200):
        k = int(rng.integers(1, 12))
        pages = rng.choice(64, size=k, replace=False)
        sel = np.sort(np.concatenate([p * 4 + rng.integers(0, 4, size=2) for p in pages]))
        victims, missed, ovf = c.resolve([sel])
        assert not ovf and len(set(victims)) == len(victims) == len(missed)
        for p in pages:
            s = c.page_table[p]
            assert s >= 0 and c.slot_page[s] == p and c.slot_stamp[s] == c.epoch
        for s, p in enumerate(c.slot_page):
            if p >= 0:
                assert c.page_table[p] == s
        assert sum(1 for x in c.page_table if x >= 0) <= 12
        assert c.rows(sel) == [c.page_table[x // 4] * 4 + x % 4 for x in sel]
