"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, call the library
through its C ABI, and compare with the fp64 oracle at the tolerances of the spec
(O max abs error 2e-3, per-row LSE abs error 1e-3; empty rows exactly O=0, LSE=-inf)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import rkv_inputs as gen

O_TOL = 2e-3
LSE_TOL = 1e-3


def step(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault still identifies it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def pinned(a: np.ndarray):
    """A freshly allocated pinned host tensor holding a copy of `a`."""
    torch = torch_mod()
    src = torch.from_numpy(np.ascontiguousarray(a))
    t = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
    t.copy_(src)
    return t


def pageable(a: np.ndarray):
    """An ordinary (pageable) host tensor holding a copy of `a`."""
    torch = torch_mod()
    return torch.from_numpy(np.array(a, copy=True))


def assert_close(O, L, Oref, Lref, o_tol=O_TOL, lse_tol=LSE_TOL, what=""):
    O = np.asarray(O, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    assert O.shape == Oref.shape, (O.shape, Oref.shape)
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    err = np.abs(O - Oref).max() if O.size else 0.0
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isfinite(L), fin), f"{what}: empty-row pattern differs"
    assert np.all(L[~fin] == -np.inf)
    lerr = np.abs(L[fin] - Lref[fin]).max() if fin.any() else 0.0
    assert err <= o_tol, f"{what}: O max abs err {err:.3e} > {o_tol}"
    assert lerr <= lse_tol, f"{what}: LSE max abs err {lerr:.3e} > {lse_tol}"
    return err, lerr


def oracle_decode(w, mask=None, heads=None, softcap=0.0):
    """fp64 oracle of a window/tail workload dict from rkv_inputs.make_workload.
    heads: optional list of KV heads to restrict to (full-size sampling)."""
    q = oracle.q_values(w["q"])
    gqa = w["n_head"] // w["n_head_kv"]
    m = None if mask is None else np.asarray(mask, dtype=np.float64)
    if heads is None:
        k = oracle.kv_values(w["k_type"], w["k"])
        v = oracle.kv_values(w["v_type"], w["v"])
        return oracle.attention(q, k, v, w["scale"], m, softcap)
    outs = {}
    for g in heads:
        k = oracle.kv_values(w["k_type"], w["k"][:, g:g + 1])
        v = oracle.kv_values(w["v_type"], w["v"][:, g:g + 1])
        O, L = oracle.attention(q[g * gqa:(g + 1) * gqa], k, v, w["scale"], m, softcap)
        outs[g] = (O, L)
    return outs


class Runner:
    """Holds one library context and runs the entry points on numpy inputs."""

    def __init__(self):
        import tiered_kv_cache_split_amd as rkv
        self.rkv = rkv
        self.ctx = rkv.Context(0)
        # the tests lift every pinned tail under the automatic lift mode; the in-place read
        # the automatic mode gives small decode tails is tested where it is switched back on
        self.ctx.set_direct_tail_max(0)

    def decode(self, w, wc=None, tile_kv=None, tail="host", mask=None, layout="cell", prefill=False,
               q_pos0=-1, stream=None, keep=None):
        torch = torch_mod()
        rkv = self.rkv
        wc = w["wc"] if wc is None else wc
        tile_kv = w["tile_kv"] if tile_kv is None else tile_kv
        n_head, n_q = w["n_head"], w["q"].shape[1]
        q = dev(w["q"])
        kc, vc = w["k"], w["v"]
        if layout == "head":
            kc = np.ascontiguousarray(np.transpose(kc, (1, 0, 2)))
            vc = np.ascontiguousarray(np.transpose(vc, (1, 0, 2)))
            kwin, vwin = kc[:, :wc], vc[:, :wc]
            ktl, vtl = kc[:, wc:], vc[:, wc:]
        else:
            kwin, vwin = kc[:wc], vc[:wc]
            ktl, vtl = kc[wc:], vc[wc:]
        tensors = {}
        kd = vd = ktd = vtd = None
        if wc > 0:
            tensors["kw"], tensors["vw"] = dev(np.ascontiguousarray(kwin)), dev(np.ascontiguousarray(vwin))
            kd = rkv.kv_desc(tensors["kw"], w["k_type"], layout)
            vd = rkv.kv_desc(tensors["vw"], w["v_type"], layout)
        n_tail = ktl.shape[0] if layout == "cell" else ktl.shape[1]
        if tail is not None and n_tail > 0:
            mk = {"host": pinned, "device": dev, "pageable": pageable}[tail]
            tensors["kt"], tensors["vt"] = mk(np.ascontiguousarray(ktl)), mk(np.ascontiguousarray(vtl))
            ktd = rkv.kv_desc(tensors["kt"], w["k_type"], layout)
            vtd = rkv.kv_desc(tensors["vt"], w["v_type"], layout)
        md = None
        if mask is not None:
            tensors["m"] = dev(np.asarray(mask, dtype=np.float16))
            md = rkv.mask_desc(tensors["m"])
        o = torch.empty((n_q, n_head, w.get("dv", w.get("d", 128))), dtype=torch.float32, device="cuda")
        lse = torch.empty((n_q, n_head), dtype=torch.float32, device="cuda")
        if prefill:
            self.ctx.attn_prefill(rkv.q_desc(q), kd, vd, ktd, vtd, md, wc, tile_kv, w["scale"], q_pos0, o, lse,
                                  stream=stream)
        else:
            self.ctx.attn_decode(rkv.q_desc(q), kd, vd, ktd, vtd, md, wc, tile_kv, w["scale"], o, lse,
                                 stream=stream)
        if keep is not None:
            keep.append((q, tensors))
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()

    def rows(self, w, mask="given", rows=None):
        torch = torch_mod()
        rkv = self.rkv
        q = dev(w["q"])
        kp, vp = dev(w["k"]), dev(w["v"])
        kvr = dev(np.ascontiguousarray(w["kv_rows"] if rows is None else rows, dtype=np.int32))
        m = w["mask"] if isinstance(mask, str) and mask == "given" else mask
        mt = None if m is None else dev(np.asarray(m, dtype=np.float16))
        n_seq, n_head, n_q, _ = w["q"].shape
        n_kv = kvr.shape[1]
        o = torch.empty((n_seq, n_q, n_head, w.get("dv", w.get("d", 128))), dtype=torch.float32, device="cuda")
        lse = torch.empty((n_seq, n_q, n_head), dtype=torch.float32, device="cuda")
        self.ctx.attn_rows(rkv.q_desc(q), rkv.kv_desc(kp, w["k_type"]), rkv.kv_desc(vp, w["v_type"]), kvr, n_kv,
                           rkv.mask_desc(mt), w["scale"], o, lse)
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()


def oracle_rows(w, mask="given", rows=None, softcap=0.0):
    q = np.stack([oracle.q_values(w["q"][b]) for b in range(w["q"].shape[0])])
    k = oracle.kv_values(w["k_type"], w["k"])
    v = oracle.kv_values(w["v_type"], w["v"])
    m = w["mask"] if isinstance(mask, str) and mask == "given" else mask
    mm = None if m is None else np.asarray(m, dtype=np.float64)[:, 0]
    return oracle.attention_rows(q, k, v, w["kv_rows"] if rows is None else rows, w["scale"], mm, softcap)
