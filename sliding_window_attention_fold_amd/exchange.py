"""Python binding of the exchange part of libnbattn (include/nbexchange.h):
argument marshalling only.

Mirrors the NeMo AutoModel ``blockdiag_cp.exchange`` page: the global
left-halo plan and the per-(source, destination) all-to-all-v plan computed
from replicated document ids, and ``_NeededKVExchange`` (forward: every rank
receives its contiguous needed K/V range; backward: index_add of every rank's
gradient onto the source tokens), here emulated for all ranks on one device:
rank ``r``'s chunk is the slice ``[r L, (r + 1) L)`` of one global tensor.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _lib

__all__ = ["ExchangePlan", "exchange_plan", "send_index", "needed_gather", "needed_scatter_add",
           "NeededKVExchange", "needed_kv_exchange"]

_DTYPES = {torch.bfloat16: _lib.NB_BF16, torch.float32: _lib.NB_F32}
_HDR = 8


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class ExchangePlan:
    """Device plan buffer plus the host copy every rank would hold."""

    buf: torch.Tensor        # int32, layout in include/nbexchange.h
    cp_size: int
    N: int
    L: int
    use_halo: bool
    halo_size: int
    total: int               # tokens received over all ranks
    s_first: np.ndarray      # [P]
    real_end: np.ndarray     # [P]
    back: np.ndarray         # [P]
    splits: np.ndarray       # [P, P]: splits[s, r] tokens source s sends destination r

    @property
    def recv_len(self) -> np.ndarray:
        return self.real_end - self.s_first


def exchange_plan(doc_ids: torch.Tensor, cp_size: int, pad_mask: Optional[torch.Tensor] = None) -> ExchangePlan:
    """Plan from replicated ``doc_ids`` ``[B, N]`` (int32, on the device).

    Synchronises once to read the plan back (the ranks' buffer sizes)."""
    if doc_ids.dim() == 1:
        doc_ids = doc_ids[None]
    if doc_ids.dtype != torch.int32 or not doc_ids.is_cuda:
        raise ValueError("doc_ids must be an int32 device tensor")
    doc_ids = doc_ids.contiguous()
    B, N = doc_ids.shape
    pm = None
    if pad_mask is not None:
        pm = (pad_mask if pad_mask.dim() == 2 else pad_mask[None]).to(torch.uint8).contiguous()
    lib = _lib.load()
    n = lib.nb_exchange_plan_elems(cp_size)
    if n == 0:
        raise ValueError(f"cp_size {cp_size} outside [1, {_lib.NB_XCH_MAX_RANKS}]")
    buf = torch.empty((n,), dtype=torch.int32, device=doc_ids.device)
    _lib.check(lib.nb_exchange_plan(_ptr(doc_ids), _ptr(pm), B, N, cp_size, _ptr(buf), n,
                                    _stream(doc_ids.device)), "nb_exchange_plan")
    h = buf.cpu().numpy().astype(np.int64)
    P = cp_size
    o = _HDR
    return ExchangePlan(buf, P, N, int(h[2]), bool(h[0]), int(h[1]), int(h[4]),
                        h[o:o + P], h[o + P:o + 2 * P], h[o + 2 * P:o + 3 * P],
                        h[o + 3 * P:o + 3 * P + P * P].reshape(P, P))


def send_index(plan: ExchangePlan) -> List[torch.Tensor]:
    """Every source's local gather index (the pieces for destinations 0, 1, ...)."""
    lib = _lib.load()
    n = lib.nb_exchange_send_index_elems(plan.cp_size, plan.N)
    out = torch.empty((n,), dtype=torch.int32, device=plan.buf.device)
    _lib.check(lib.nb_exchange_send_index(_ptr(plan.buf), plan.cp_size, plan.N, _ptr(out), n,
                                          _stream(out.device)), "nb_exchange_send_index")
    counts = plan.splits.sum(axis=1)
    return [out[s * plan.N:s * plan.N + int(counts[s])] for s in range(plan.cp_size)]


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if (t is None or t.numel() == 0) else t.data_ptr()
    return arr


def needed_gather(x: torch.Tensor, plan: ExchangePlan) -> List[torch.Tensor]:
    """``x`` ``[B, C, N, D]`` global -> every rank's received range ``[B, C, R_r, D]``."""
    B, C, N, D = x.shape
    if N != plan.N or x.dtype not in _DTYPES:
        raise ValueError("x must be [B, C, N, D] bf16/float32 with the plan's N")
    x = x.contiguous()
    recv = [torch.empty((B, C, int(R), D), dtype=x.dtype, device=x.device) for R in plan.recv_len]
    _lib.check(_lib.load().nb_exchange_gather(_ptr(x), _ptr(plan.buf), B, C, N, D, plan.cp_size, _DTYPES[x.dtype],
                                              _ptr_array(recv), _stream(x.device)), "nb_exchange_gather")
    return recv


def needed_scatter_add(grads: Sequence[Optional[torch.Tensor]], plan: ExchangePlan, B: int, C: int, D: int,
                       dtype: torch.dtype, device) -> torch.Tensor:
    """Gradients of every rank's range -> gradient of the global ``[B, C, N, D]``."""
    if len(grads) != plan.cp_size or dtype not in _DTYPES:
        raise ValueError("one gradient (or None) per rank, bf16/float32")
    gs = []
    for r, g in enumerate(grads):
        if g is not None:
            if tuple(g.shape) != (B, C, int(plan.recv_len[r]), D) or g.dtype != dtype:
                raise ValueError(f"gradient of rank {r} has the wrong shape or dtype")
            g = g.contiguous()
        gs.append(g)
    out = torch.empty((B, C, plan.N, D), dtype=dtype, device=device)
    _lib.check(_lib.load().nb_exchange_scatter_add(_ptr_array(gs), _ptr(plan.buf), B, C, plan.N, D, plan.cp_size,
                                                   _DTYPES[dtype], _ptr(out), _stream(out.device)),
               "nb_exchange_scatter_add")
    return out


class NeededKVExchange(torch.autograd.Function):
    """``_NeededKVExchange`` for every rank at once: forward gathers each rank's
    needed range, backward index_adds the ranks' gradients onto the tokens."""

    @staticmethod
    def forward(ctx, x, plan: ExchangePlan):
        ctx.plan = plan
        ctx.meta = (x.shape[0], x.shape[1], x.shape[3], x.dtype, x.device)
        return tuple(needed_gather(x, plan))

    @staticmethod
    def backward(ctx, *grads):
        B, C, D, dtype, device = ctx.meta
        return needed_scatter_add(list(grads), ctx.plan, B, C, D, dtype, device), None


def needed_kv_exchange(x: torch.Tensor, plan: ExchangePlan) -> List[torch.Tensor]:
    return list(NeededKVExchange.apply(x, plan))
