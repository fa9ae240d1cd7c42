"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them element by element.

Tolerances: |x - r| <= atol + rtol * |r| for every element, with
atol = rtol = 2e-2 for bfloat16 and 1e-4 for the float32 debug path; -inf LSE
must match exactly, and outputs the oracle makes structurally zero (padding
rows of O and dQ, keys no query attends, owners not attended) must be exact
zeros.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from oracle import nbattn_oracle as orc
import sliding_window_attention_fold_amd as nb
from sliding_window_attention_fold_amd import workloads as wl

TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-4, 1e-4)}


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(name, x, ref, dtype, mask=None):
    atol, rtol = TOL[dtype]
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (name, x.shape, ref.shape)
    if mask is not None:
        x, ref = x[mask], ref[mask]
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(x), ninf), f"{name}: -inf pattern differs"
    x, ref = x[~ninf], ref[~ninf]
    assert np.isfinite(x).all(), f"{name}: non-finite values"
    err = np.abs(x - ref)
    bad = err > atol + rtol * np.abs(ref)
    big = np.abs(ref) > atol
    rel = (err[big] / np.abs(ref[big])).max() if big.any() else 0.0
    assert not bad.any(), (f"{name}: {int(bad.sum())}/{bad.size} outside tolerance; max abs {err.max():.3e} "
                           f"max rel {rel:.3e}")
    return float(err.max()) if err.size else 0.0


@dataclass
class Inputs:
    ids: np.ndarray
    pad: Optional[np.ndarray]
    folded: np.ndarray
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    L: int
    S: int
    window: int
    owner_off: list
    owners: list
    cp_rank: int
    cp_size: int


def workload_inputs(w: wl.Workload, dtype: str) -> Inputs:
    dm = wl.make_doc_map(w)
    q, k, v, do = wl.make_tensors(w, dm.S, dtype)
    return Inputs(dm.doc_ids, dm.pad_mask, orc.fold_pad(dm.doc_ids, dm.pad_mask), q, k, v, do, w.L, dm.S,
                  w.window, dm.owner_off, dm.owners, w.cp_rank, w.cp_size)


def custom_inputs(ids, pad, Hq, Hkv, D, L, window, dtype, seed, owner_off=None, outliers=False):
    """Inputs with an explicit doc map (edge cases); tensors drawn like the workloads."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    B, S = ids.shape
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, Hq, L, D), generator=g)
    k = torch.randn((B, Hkv, S, D), generator=g)
    v = torch.randn((B, Hkv, S, D), generator=g)
    do = torch.randn((B, Hq, L, D), generator=g)
    if outliers:
        q = torch.where(torch.rand(q.shape, generator=g) < 0.01, q * 8, q)
        k = torch.where(torch.rand(k.shape, generator=g) < 0.01, k * 8, k)
    if dtype == "bf16":
        q, k, v, do = (t.to(torch.bfloat16) for t in (q, k, v, do))
    owner_off = [0, S] if owner_off is None else owner_off
    return Inputs(ids, pad, orc.fold_pad(ids, pad), q, k, v, do, L, S, window, owner_off,
                  list(range(len(owner_off) - 1)), len(owner_off) - 2, len(owner_off) - 1)


def run_gpu(inp: Inputs, owners=True):
    dev = torch.device("cuda:0")
    ids = torch.from_numpy(inp.ids).to(dev)
    pad = None if inp.pad is None else torch.from_numpy(np.ascontiguousarray(inp.pad)).to(dev)
    seg = nb.segment_build(ids, inp.L, inp.window, pad)
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    out, saved = nb.attn_fwd(q, k, v, seg)
    table = nb.OwnerTable(inp.owner_off, inp.owners, inp.cp_rank, inp.cp_size) if owners else None
    res = nb.attn_bwd(saved, do, table)
    torch.cuda.synchronize()
    return seg, out, saved.lse, res


def check_segments(seg, inp: Inputs):
    ref = orc.segments_reference(inp.folded, inp.L, inp.window)
    h = seg.header_host()
    n = ref["n_seg"]
    assert h["n_seg"] == n and h["max_q"] == ref["max_q"] and h["max_k"] == ref["max_k"]
    assert h["status"] == ref["status"] and h["lo"] == ref["lo"]
    assert h["n_real"] == int(orc.real_rows(inp.folded, inp.L).sum())
    assert np.array_equal(seg.folded.cpu().numpy(), inp.folded)
    for key, m in (("cu_q", n + 1), ("cu_k", n + 1), ("q_row0", n), ("k_row0", n)):
        assert np.array_equal(getattr(seg, key).cpu().numpy()[:m], ref[key][:m]), key
    for key in ("row_seg", "row_klo", "kcov_lo"):
        assert np.array_equal(getattr(seg, key).cpu().numpy(), ref[key]), key


def full_parity(inp: Inputs, dtype: str, check_bwd=True):
    """Every element of O, LSE, dQ, dK, dV against the oracle (small sizes)."""
    seg, out, lse, res = run_gpu(inp)
    check_segments(seg, inp)
    scale = inp.q.shape[-1] ** -0.5
    O, LSE = orc.attention_forward(inp.q, inp.k, inp.v, inp.folded, inp.window, scale)
    real = orc.real_rows(inp.folded, inp.L)
    assert_close("O", out.float().cpu().numpy(), O, dtype)
    assert_close("LSE", lse.cpu().numpy(), LSE, dtype)
    o_np = out.float().cpu().numpy()
    assert (o_np[~np.broadcast_to(real[:, None, :], o_np.shape[:3])] == 0).all(), "padding rows of O not 0"
    if not check_bwd:
        return
    dQ, dK, dV = orc.attention_backward(inp.q, inp.k, inp.v, inp.do, inp.folded, inp.window, scale)
    dq = res.dq.float().cpu().numpy()
    dk = res.dk.float().cpu().numpy()
    dv = res.dv.float().cpu().numpy()
    assert_close("dQ", dq, dQ, dtype)
    assert_close("dK", dk, dK, dtype)
    assert_close("dV", dv, dV, dtype)
    assert (dq[~np.broadcast_to(real[:, None, :], dq.shape[:3])] == 0).all(), "padding rows of dQ not 0"
    att = orc.key_attended(inp.folded, inp.L, inp.window)
    cov = np.broadcast_to(att[:, None, :], dk.shape[:3])
    assert (dk[~cov] == 0).all() and (dv[~cov] == 0).all(), "unattended keys not exact 0"
    _, _, attended = orc.owner_split(dK, dV, inp.owner_off, att)
    for o, rank in enumerate(inp.owners):
        assert res.attended[rank] == attended[o], (rank, res.attended[rank], attended[o])
        if not attended[o]:
            assert (res.dk_by_owner[rank].float() == 0).all() and (res.dv_by_owner[rank].float() == 0).all()
