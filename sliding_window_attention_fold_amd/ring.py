"""Python binding of the ring part of libnbattn (include/nbring.h): argument
marshalling only.

Mirrors the NeMo AutoModel ``gemma4_moe.cp_attention`` page's global-layer
ring for one rank, with every chunk resident on one device: the per-chunk
forward returning ``(out, lse)`` (own chunk causal, earlier owners'
non-causal), the ``-inf``-safe online merge and its live-row form, and the
per-chunk backward with the global merged out and lse, whose dQ contributions
are summed in fp32 and whose dK/dV are the owners' shares.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib

__all__ = ["RingSegments", "ring_segments", "chunk_fwd", "merge_", "live_rows", "merge_live_", "finalize",
           "chunk_bwd", "grad_add_", "ring_forward", "ring_backward"]

_DTYPES = {torch.bfloat16: _lib.NB_BF16, torch.float32: _lib.NB_F32}


def _s(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class RingSegments:
    """Segments of rank ``q_start / L``'s shard over the global doc map's prefix
    ``[0, q_start + L)``: row_klo holds each query row's document start in
    global positions (one buffer for every chunk)."""

    seg_buf: torch.Tensor
    folded: torch.Tensor
    B: int
    L: int
    q_start: int


def ring_segments(doc_ids: torch.Tensor, q_start: int, L: int, pad_mask: Optional[torch.Tensor] = None) -> RingSegments:
    """``doc_ids`` ``[B, N]`` int32 (the global map, on the device)."""
    if doc_ids.dim() == 1:
        doc_ids = doc_ids[None]
    B = doc_ids.shape[0]
    S = q_start + L
    if doc_ids.dtype != torch.int32 or not doc_ids.is_cuda or S > doc_ids.shape[1] or q_start < 0:
        raise ValueError("doc_ids must be an int32 device tensor [B, N] with q_start + L <= N")
    ids = doc_ids[:, :S].contiguous()
    pm = None
    if pad_mask is not None:
        pm = (pad_mask if pad_mask.dim() == 2 else pad_mask[None])[:, :S].to(torch.uint8).contiguous()
    lib = _lib.load()
    n = lib.nb_segment_buffer_elems(B, L, S)
    seg = torch.empty((n,), dtype=torch.int32, device=ids.device)
    folded = torch.empty_like(ids)
    _lib.check(lib.nb_segment_build(_p(ids), _p(pm), B, S, L, -1, _p(folded), _p(seg), n, _s(ids.device)),
               "nb_segment_build")
    return RingSegments(seg, folded, B, L, q_start)


def _dims(q, k):
    B, Hq, L, D = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != D or q.dtype not in _DTYPES or k.dtype != q.dtype:
        raise ValueError("q [B, Hq, L, D] and k/v [B, Hkv, Lk, D] of one dtype (bf16 or float32)")
    return B, Hq, k.shape[1], L, k.shape[2], D


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, segs: RingSegments, k_start: int,
              scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One chunk's ``(out, lse)`` (``_ffpa_varlen_forward_chunk``); keys at global
    positions ``k_start ..``."""
    B, Hq, Hkv, L, Lk, D = _dims(q, k)
    scale = D ** -0.5 if scale is None else float(scale)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if lse is None else lse
    _lib.check(_lib.load().nb_ring_chunk_fwd(_p(q), _p(k), _p(v), _p(out), _p(lse), _p(segs.seg_buf), B, Hq, Hkv, L,
                                             Lk, D, segs.q_start, k_start, scale, _DTYPES[q.dtype], _s(q.device)),
               "nb_ring_chunk_fwd")
    return out, lse


def merge_(out_acc: torch.Tensor, lse_acc: torch.Tensor, out_step: torch.Tensor, lse_step: torch.Tensor,
           init: bool = False) -> None:
    """In-place ``-inf``-safe merge (``_merge_ffpa_packed_chunk``); fp32 accumulators.  ``init``: the
    accumulators become the step (nothing merged yet)."""
    D = out_acc.shape[-1]
    _lib.check(_lib.load().nb_ring_merge(_p(out_acc), _p(lse_acc), _p(out_step.contiguous()), _p(lse_step),
                                         lse_acc.numel(), D, _DTYPES[out_step.dtype], int(init), _s(out_acc.device)),
               "nb_ring_merge")


def live_rows(segs: RingSegments, Lk: int, k_start: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """``(live_index [B * L] int32, n_live [1] int32)`` on the device."""
    dev = segs.seg_buf.device
    idx = torch.empty((segs.B * segs.L,), dtype=torch.int32, device=dev)
    n = torch.empty((1,), dtype=torch.int32, device=dev)
    _lib.check(_lib.load().nb_ring_live_rows(_p(segs.seg_buf), segs.B, segs.L, Lk, segs.q_start, k_start, _p(idx),
                                             _p(n), _s(dev)), "nb_ring_live_rows")
    return idx, n


def merge_live_(out_acc, lse_acc, out_step, lse_step, live_index, n_live, n_live_max: Optional[int] = None) -> None:
    """``_merge_live_chunk_``: merge at the listed rows of every head."""
    B, H, L, D = out_acc.shape
    n_max = live_index.numel() if n_live_max is None else int(n_live_max)
    _lib.check(_lib.load().nb_ring_merge_live(_p(out_acc), _p(lse_acc), _p(out_step.contiguous()), _p(lse_step),
                                              _p(live_index), _p(n_live), n_max, B, H, L, D,
                                              _DTYPES[out_step.dtype], _s(out_acc.device)), "nb_ring_merge_live")


def finalize(out_acc: torch.Tensor, dtype: torch.dtype, with_resid: bool = True):
    """``(out, resid)``: the merged output rounded to ``dtype`` and, for bf16, its rounding-residual codes
    (int8, one per element; None for float32)."""
    out = torch.empty(out_acc.shape, dtype=dtype, device=out_acc.device)
    resid = (torch.empty(out.shape, dtype=torch.int8, device=out.device)
             if with_resid and dtype == torch.bfloat16 else None)
    D = out_acc.shape[-1]
    _lib.check(_lib.load().nb_ring_finalize(_p(out_acc), _p(out), _p(resid), out_acc.numel() // D, D,
                                            _DTYPES[dtype], _s(out_acc.device)), "nb_ring_finalize")
    return out, resid


def _ws_bytes(lib, B, Hq, Hkv, L, Lk, D, dt, stored_ds):
    # D = 512 has only the stored-dS form
    return (lib.nb_ring_chunk_bwd_workspace_bytes(B, Hq, Hkv, L, Lk, D, dt) if stored_ds or D >= 512
            else lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, Lk, D, dt))


def chunk_bwd(dout, q, k, v, o, o_resid, lse, segs: RingSegments, k_start: int, scale: Optional[float] = None,
              ws: Optional[torch.Tensor] = None, dq_acc: Optional[torch.Tensor] = None, dq_init: bool = False,
              delta_ready: bool = False, stored_ds: bool = False):
    """One chunk's ``(dQ contribution, dK, dV)`` with the global out/lse
    (``_ffpa_varlen_backward_chunk``).  With ``dq_acc`` (fp32) the contribution
    is added to it (``dq_init``: written) and returned in its place;
    ``delta_ready``: ``ws`` holds Delta from an earlier call.  ``stored_ds``: a
    workspace with room for dS (at D = 256 the library then stores dS and forms
    dQ from it whenever ``ws`` is that large; without a window the band spans
    the chunk, which pays only where few rows reach it).  At D = 512 the
    stored-dS form is the only one and its workspace is always given."""
    B, Hq, Hkv, L, Lk, D = _dims(q, k)
    scale = D ** -0.5 if scale is None else float(scale)
    lib = _lib.load()
    dt = _DTYPES[q.dtype]
    need = _ws_bytes(lib, B, Hq, Hkv, L, Lk, D, dt, stored_ds)
    if ws is None or ws.numel() < need:
        if delta_ready:
            raise ValueError("delta_ready needs the workspace of the earlier call")
        ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
    flags = _lib.NB_RING_DELTA_READY if delta_ready else 0
    if dq_acc is not None:
        if dq_acc.dtype != torch.float32 or tuple(dq_acc.shape) != tuple(q.shape):
            raise ValueError("dq_acc must be float32 [B, Hq, L, D]")
        dq = dq_acc
        flags |= _lib.NB_RING_DQ_F32_SET if dq_init else _lib.NB_RING_DQ_F32_ADD
    else:
        dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    args = [t.contiguous() for t in (dout, q, k, v, o)]
    _lib.check(lib.nb_ring_chunk_bwd(*[_p(t) for t in args], _p(o_resid), _p(lse), _p(segs.seg_buf), B, Hq, Hkv, L,
                                     Lk, D, segs.q_start, k_start, scale, dt, _p(dq), _p(dk), _p(dv), flags, _p(ws),
                                     ws.numel(), _s(q.device)), "nb_ring_chunk_bwd")
    return dq, dk, dv


def grad_add_(acc: torch.Tensor, src: torch.Tensor, init: bool = False) -> None:
    """``acc += src`` in fp32 (``_grad_add_live_`` over every row); ``init``: ``acc = src``."""
    _lib.check(_lib.load().nb_ring_grad_add(_p(acc), _p(src.contiguous()), acc.numel(), _DTYPES[src.dtype],
                                            int(init), _s(acc.device)), "nb_ring_grad_add")


def ring_forward(q: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor],
                 segs: RingSegments, chunk_starts: Sequence[int], scale: Optional[float] = None,
                 live: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """``_run_gemma4_cp_ffpa_varlen_ring_forward`` for one rank: the chunks in
    visiting order (own chunk first), ``chunk_starts`` their global first
    positions.  Returns the fp32 ``(out, lse)``; with ``live`` the chunks after
    the first merge at their live rows only."""
    B, Hq, L, D = q.shape
    out_acc = torch.empty((B, Hq, L, D), dtype=torch.float32, device=q.device)
    lse_acc = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    out_step = torch.empty_like(q)
    lse_step = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    for c, (k, v, ks) in enumerate(zip(k_chunks, v_chunks, chunk_starts)):
        chunk_fwd(q, k, v, segs, ks, scale, out_step, lse_step)
        if live and c > 0:
            idx, n = live_rows(segs, k.shape[2], ks)
            merge_live_(out_acc, lse_acc, out_step, lse_step, idx, n)
        else:
            merge_(out_acc, lse_acc, out_step, lse_step, init=c == 0)
    return out_acc, lse_acc


def ring_backward(dout, q, k_chunks, v_chunks, out, out_resid, lse, segs: RingSegments, chunk_starts,
                  scale: Optional[float] = None, stored_ds: bool = False):
    """Every chunk's backward with the global out/lse: ``(dQ fp32, [dK_c], [dV_c])``."""
    B, Hq, L, D = q.shape
    dq_acc = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dks: List[torch.Tensor] = []
    dvs: List[torch.Tensor] = []
    lib = _lib.load()
    need = max(_ws_bytes(lib, B, Hq, k.shape[1], L, k.shape[2], D, _DTYPES[q.dtype], stored_ds) for k in k_chunks)
    ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
    for c, (k, v, ks) in enumerate(zip(k_chunks, v_chunks, chunk_starts)):
        _, dk, dv = chunk_bwd(dout, q, k, v, out, out_resid, lse, segs, ks, scale, ws, dq_acc=dq_acc,
                              dq_init=c == 0, delta_ready=c > 0, stored_ds=stored_ds)
        dks.append(dk)
        dvs.append(dv)
    return dq_acc, dks, dvs
