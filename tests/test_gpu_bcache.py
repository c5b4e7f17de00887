"""The device-side block cache (rkv_bcache_*) against a resident cache and the CLOCK oracle.

Strata's own parity test for KV streaming (Strata compare, "KV streaming for the QSA layers",
``kv_stream_parity``) is the model: output through the streamed cache must equal the fully
resident output bitwise, the map must be its own inverse and the counters consistent.  Here each
call also checks the residency decisions against ``oracle.ClockCache``: the set of resident
pages, the victim slots, the hand and the counters (which missed page goes to which victim
slot is the device's claim order; the oracle adopts it before the next call)."""
import numpy as np
import pytest

import oracle
import rkv_inputs as gen
from rkv_testutil import assert_close, dev, pinned, step

pytestmark = pytest.mark.gpu

PS = 16  # cells per page


def make_cache(rng, n_cells, n_head_kv, k_type, v_type, outliers=False):
    if k_type == gen.TYPE_F16:
        kx = rng.standard_normal((n_cells, n_head_kv, 128)).astype(np.float32)
        if outliers:
            kx[::17] *= 30.0
        k = gen.pack_f16(kx)
    else:
        k = gen.pack_raw_edge(rng, k_type, (n_cells, n_head_kv), 128)
    if v_type == gen.TYPE_F16:
        v = gen.pack_f16(rng.standard_normal((n_cells, n_head_kv, 128)).astype(np.float32))
    else:
        v = gen.pack_raw_edge(rng, v_type, (n_cells, n_head_kv), 128)
    return k, v


def selection(rng, n_pages, n_seq, pages_per_seq, width):
    """Per sequence: cells drawn from a few random pages, ascending, padded with -1."""
    sel = np.full((n_seq, width), -1, np.int32)
    for b in range(n_seq):
        pages = rng.choice(n_pages, size=pages_per_seq, replace=False)
        cells = np.unique(np.concatenate([p * PS + rng.choice(PS, size=int(rng.integers(1, PS + 1)), replace=False)
                                          for p in pages]))[:width]
        sel[b, :len(cells)] = cells
    return sel


class Harness:
    def __init__(self, n_cells=4096, n_head_kv=8, n_head=32, n_slots=48, k_type=gen.TYPE_F16, v_type=gen.TYPE_F16,
                 seed=3, outliers=False, n_seq=2):
        import torch
        import tiered_kv_cache_split_amd as rkv
        self.rkv, self.torch = rkv, torch
        rng = np.random.default_rng(seed)
        self.rng = rng
        self.k, self.v = make_cache(rng, n_cells, n_head_kv, k_type, v_type, outliers)
        self.k_type, self.v_type = k_type, v_type
        self.kh, self.vh = pinned(self.k), pinned(self.v)          # authoritative host copy
        self.kd, self.vd = dev(self.k), dev(self.v)                 # resident reference
        self.bc = rkv.BlockCache(self.kh, self.vh, k_type, v_type, PS, n_slots)
        self.ctx = rkv.Context(0)
        self.n_pages, self.n_slots, self.n_head, self.n_head_kv, self.n_seq = n_cells // PS, n_slots, n_head, n_head_kv, n_seq
        self.q = rng.standard_normal((n_seq, n_head, 1, 128)).astype(np.float16)
        self.qd = dev(self.q)
        self.model = oracle.ClockCache(self.n_pages, n_slots, PS)

    def attn(self, k_desc, v_desc, rows_dev, width, mask_dev):
        torch, rkv = self.torch, self.rkv
        o = torch.empty((self.n_seq, 1, self.n_head, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((self.n_seq, 1, self.n_head), dtype=torch.float32, device="cuda")
        self.ctx.attn_rows(rkv.q_desc(self.qd), k_desc, v_desc, rows_dev, width, rkv.mask_desc(mask_dev),
                           1 / np.sqrt(128), o, lse)
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()

    def call(self, sel, check_oracle=False):
        torch, rkv = self.torch, self.rkv
        width = sel.shape[1]
        seld = dev(sel)
        rows = torch.empty_like(seld)
        self.bc.resolve(seld, rows)
        mask = np.where(sel[:, None, None, :] >= 0, 0.0, -np.inf).astype(np.float16)
        maskd = dev(mask)
        kp, vp = self.bc.pools()
        O_s, L_s = self.attn(kp, vp, rows, width, maskd)
        O_r, L_r = self.attn(rkv.kv_desc(self.kd, self.k_type), rkv.kv_desc(self.vd, self.v_type), seld, width, maskd)
        # streamed == resident, bit for bit
        assert np.array_equal(O_s.view(np.uint32), O_r.view(np.uint32)) and np.array_equal(L_s.view(np.uint32), L_r.view(np.uint32))
        # residency decisions against the policy
        prev_resident = {p for p, s in enumerate(self.model.page_table) if s >= 0}
        victims, missed, ovf = self.model.resolve([list(x) for x in sel])
        pt, sp = self.bc.map_arrays()
        c = self.bc.counters()
        resident = {p for p, s in enumerate(pt) if s >= 0}
        assert resident == {p for p, s in enumerate(self.model.page_table) if s >= 0}
        assert sorted(int(pt[p]) for p in missed) == sorted(victims)
        assert (c["hand"], c["epoch"], c["misses"], c["lookups"], c["calls"]) == \
            (self.model.hand, self.model.epoch, self.model.misses, self.model.lookups, self.model.calls)
        assert c["last_misses"] == len(victims) and bool(c["overflow"]) == self.model.overflow
        # the map is its own inverse; nothing left claimed
        assert np.all(pt >= -1)
        for s, p in enumerate(sp):
            if p >= 0:
                assert pt[p] == s
        for p, s in enumerate(pt):
            if s >= 0:
                assert sp[s] == p
        self.model.adopt(pt, sp)
        assert list(rows.cpu().numpy().reshape(-1)) == [r for b in range(sel.shape[0]) for r in self.model.rows(sel[b])]
        if check_oracle:
            q = np.stack([oracle.q_values(self.q[b]) for b in range(self.n_seq)])
            kk = oracle.kv_values(self.k_type, self.k)
            vv = oracle.kv_values(self.v_type, self.v)
            Oref, Lref = oracle.attention_rows(q, kk, vv, sel, 1 / np.sqrt(128), mask[:, 0].astype(np.float64))
            assert_close(O_s, L_s, Oref, Lref, what="block cache vs fp64 oracle")
        return prev_resident, resident


def test_streamed_equals_resident_over_many_calls():
    h = Harness()
    step("block cache f16: 30 calls, 48 slots, 256 pages")
    for t in range(30):
        sel = selection(h.rng, h.n_pages, h.n_seq, int(h.rng.integers(2, 12)), 12 * PS)
        h.call(sel, check_oracle=(t in (0, 29)))
    assert h.bc.counters()["misses"] > h.n_slots  # evictions happened


def test_repeated_selection_hits():
    h = Harness(seed=5)
    sel = selection(h.rng, h.n_pages, h.n_seq, 6, 6 * PS)
    step("block cache: same selection twice, all hits the second time")
    h.call(sel)
    misses = h.bc.counters()["misses"]
    h.call(sel)
    c = h.bc.counters()
    assert c["misses"] == misses and c["last_misses"] == 0


@pytest.mark.parametrize("outliers", [False, True])
def test_quant_cache_and_outlier_keys(outliers):
    """q8_0 K / q4_0 V edge bytes (or binary16 K with every 17th key x30) through the cache."""
    kt = gen.TYPE_F16 if outliers else gen.TYPE_Q8_0
    vt = gen.TYPE_F16 if outliers else gen.TYPE_Q4_0
    h = Harness(n_cells=2048, n_head_kv=4, n_head=16, n_slots=24, k_type=kt, v_type=vt, seed=9, outliers=outliers)
    step(f"block cache types {kt}/{vt} outliers {outliers}")
    for t in range(8):
        sel = selection(h.rng, h.n_pages, h.n_seq, int(h.rng.integers(2, 6)), 6 * PS)
        h.call(sel, check_oracle=(t == 7))


def test_write_through_append():
    """Appends land in the host copy always and in the slot only while the page is resident; the
    next read through the cache equals the resident read of the updated cache."""
    h = Harness(seed=11)
    torch = h.torch
    sel = selection(h.rng, h.n_pages, h.n_seq, 4, 4 * PS)
    h.call(sel)
    pt, _ = h.bc.map_arrays()
    res_cell = int(sel[0, 0])                                   # page resident now
    absent_page = int(np.flatnonzero(pt < 0)[0])
    abs_cell = absent_page * PS + 3                             # page absent now
    step("block cache append: resident and absent pages")
    for cell in (res_cell, abs_cell):
        kx = h.rng.standard_normal((h.n_head_kv, 128)).astype(np.float32)
        vx = h.rng.standard_normal((h.n_head_kv, 128)).astype(np.float32)
        kb, vb = gen.pack_f16(kx), gen.pack_f16(vx)
        h.bc.append(dev(kb), dev(vb), cell)
        torch.cuda.synchronize()
        assert np.array_equal(h.kh[cell].numpy(), kb) and np.array_equal(h.vh[cell].numpy(), vb)
        h.k[cell], h.v[cell] = kb, vb
        h.kd[cell] = torch.from_numpy(kb).cuda()
        h.vd[cell] = torch.from_numpy(vb).cuda()
    sel2 = sel.copy()
    cells1 = np.unique(np.concatenate([sel[1][sel[1] >= 0], [abs_cell - 3, abs_cell, abs_cell + 1]]))[:sel.shape[1]]
    sel2[1] = -1
    sel2[1, :len(cells1)] = cells1
    h.call(sel2, check_oracle=True)


def test_overflow_is_reported():
    """One call naming more pages than slots: the first n_slots pages placed, the rest absent with
    rows -1, the overflow counter set; the output of the placed rows stays correct."""
    import torch
    h = Harness(n_slots=8, seed=13, n_seq=1)
    sel = (np.arange(12, dtype=np.int32) * PS)[None, :]  # 12 pages, 8 slots
    step("block cache overflow: 12 pages, 8 slots")
    seld = dev(sel)
    rows = torch.empty_like(seld)
    h.bc.resolve(seld, rows)
    c = h.bc.counters()
    assert c["overflow"] == 1 and c["last_misses"] == 8
    r = rows.cpu().numpy()[0]
    assert (r >= 0).sum() == 8 and (r == -1).sum() == 4
    pt, sp = h.bc.map_arrays()
    assert (pt >= 0).sum() == 8 and np.all(pt >= -1)
    assert sorted(sp[sp >= 0].tolist()) == sorted(np.flatnonzero(pt >= 0).tolist())
