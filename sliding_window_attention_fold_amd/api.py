"""Python binding of libnbattn: argument marshalling only.

PyTorch provides device memory and the stream; every step of the computation
runs in the HIP kernels behind the C-ABI.  The functions mirror the NeMo
AutoModel ``cp_local_ring`` page: ``sliding_ring_compute_fa_fwd`` (forward,
returns ``(out, saved)``), ``sliding_ring_compute_fa_bwd`` (backward, returns
``dQ`` and per-owner dK/dV maps) and ``_owner_grad_dict`` (the full
``owner -> grad`` map with zeros for owners the shard did not attend), with the
per-step segment build of ``_cached_sliding_segments`` made explicit: the caller
builds :class:`Segments` once per step and reuses it for every layer and both
passes.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from collections.abc import Mapping
from typing import Dict, List, NamedTuple, Optional

import torch

from . import _lib

__all__ = ["Segments", "OwnerTable", "OwnerFlags", "Saved", "BwdResult", "segment_build", "attn_fwd", "attn_bwd",
           "NeighbourhoodAttention", "neighbourhood_attention", "KvChunk", "ChunkSaved", "attn_fwd_chunks",
           "attn_bwd_chunks", "ring_window_chunks"]

_DTYPES = {torch.bfloat16: _lib.NB_BF16, torch.float32: _lib.NB_F32}


def _stream_ptr(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


@dataclass
class Segments:
    """Device segment buffer of one shard (built once per step, reused by every layer)."""

    folded: torch.Tensor   # [B, S] int32, doc ids with padding folded to 0
    buf: torch.Tensor      # int32 segment buffer (layout in include/nbattn.h)
    B: int
    L: int
    S: int
    window: int

    def _view(self, fn: str, n: int) -> torch.Tensor:
        off = getattr(_lib.load(), fn)(self.B, self.L)
        return self.buf[off:off + n]

    @property
    def header(self) -> torch.Tensor:
        return self.buf[:_lib.NB_SEG_HEADER]

    def header_host(self) -> Dict[str, int]:
        """Synchronising read of the header (debug)."""
        h = (ctypes.c_int32 * _lib.NB_SEG_HEADER)()
        _lib.check(_lib.load().nb_segment_header(_ptr(self.buf), ctypes.cast(h, ctypes.c_void_p),
                                                 _stream_ptr(self.buf.device)), "nb_segment_header")
        return {k: int(h[i]) for k, i in _lib.HDR.items()}

    @property
    def cu_q(self):
        return self._view("nb_segment_offset_cu_q", self.B * self.L + 1)

    @property
    def cu_k(self):
        return self._view("nb_segment_offset_cu_k", self.B * self.L + 1)

    @property
    def q_row0(self):
        return self._view("nb_segment_offset_q_row0", self.B * self.L)

    @property
    def k_row0(self):
        return self._view("nb_segment_offset_k_row0", self.B * self.L)

    @property
    def row_seg(self):
        return self._view("nb_segment_offset_row_seg", self.B * self.L)

    @property
    def row_klo(self):
        return self._view("nb_segment_offset_row_klo", self.B * self.L)

    @property
    def kcov_lo(self):
        return self._view("nb_segment_offset_kcov_lo", self.B)

    @property
    def fwd_order(self):
        """Per batch row, the forward's 128-row query tiles in launch order (longest band first)."""
        return self._view("nb_segment_offset_fwd_order", self.B * ((self.L + 127) // 128))


def segment_build(nb_ids: torch.Tensor, L: int, window: int = -1,
                  pad_mask: Optional[torch.Tensor] = None) -> Segments:
    """Fold padding and build the per-document varlen segments on the device (no host sync)."""
    lib = _lib.load()
    _need(nb_ids.is_cuda and nb_ids.dtype == torch.int32 and nb_ids.dim() == 2 and nb_ids.is_contiguous(),
          "nb_ids must be a contiguous [B, S] int32 device tensor")
    B, S = nb_ids.shape
    if pad_mask is not None:
        _need(pad_mask.is_cuda and pad_mask.dtype == torch.uint8 and tuple(pad_mask.shape) == (B, S)
              and pad_mask.is_contiguous(), "pad_mask must be a contiguous [B, S] uint8 device tensor")
    n = lib.nb_segment_buffer_elems(B, L, S)
    _need(n > 0, f"invalid sizes B={B} L={L} S={S}")
    folded = torch.empty((B, S), dtype=torch.int32, device=nb_ids.device)
    buf = torch.empty((n,), dtype=torch.int32, device=nb_ids.device)
    w = -1 if window is None or window < 0 else int(window)
    _lib.check(lib.nb_segment_build(_ptr(nb_ids), _ptr(pad_mask), B, S, L, w, _ptr(folded), _ptr(buf), n,
                                    _stream_ptr(nb_ids.device)), "nb_segment_build")
    return Segments(folded, buf, B, L, S, w)


@dataclass
class OwnerTable:
    """Owner chunks of the neighbourhood, ascending (``_concat_neighborhood`` order).

    ``offsets`` has ``len(owners) + 1`` entries from 0 to S.  ``cp_rank``,
    ``cp_size`` and ``n_prior`` give the full map ``_owner_grad_dict`` returns:
    every owner ``(cp_rank - d) % cp_size`` for ``d`` in ``0..n_prior``, with zeros
    for owners outside the neighbourhood (future / wrapped).
    """

    offsets: List[int]
    owners: List[int]
    cp_rank: int = 0
    cp_size: int = 1
    n_prior: Optional[int] = None

    @staticmethod
    def ring(cp_rank: int, cp_size: int, chunk: int, n_prior: Optional[int] = None) -> "OwnerTable":
        return OwnerTable([chunk * r for r in range(cp_rank + 2)], list(range(cp_rank + 1)),
                          cp_rank, cp_size, cp_rank if n_prior is None else n_prior)

    @staticmethod
    def single(S: int) -> "OwnerTable":
        return OwnerTable([0, S], [0], 0, 1, 0)


class Saved(NamedTuple):
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    out: torch.Tensor
    out_resid: Optional[torch.Tensor]  # int8 rounding-residual codes of out (bf16 path), None for float32
    lse: torch.Tensor
    seg: Segments
    scale: float


class OwnerFlags(Mapping):
    """``owner -> attended`` read lazily from the device flags.

    The backward only enqueues work; the flags stay on the device (``flags``,
    uint8, one per owner of the table, in table order) until a value is read
    here, and only that first read synchronises.  Owners outside the
    neighbourhood (future or wrapped ring owners) are ``False`` without any
    device read."""

    def __init__(self, flags: torch.Tensor, owners: List[int], absent: List[int]):
        self.flags = flags
        self._index = {r: o for o, r in enumerate(owners)}
        self._absent = [r for r in absent if r not in self._index]
        self._host: Optional[List[int]] = None

    def __getitem__(self, rank: int) -> bool:
        if rank in self._index:
            if self._host is None:
                self._host = self.flags.tolist()
            return bool(self._host[self._index[rank]])
        if rank in self._absent:
            return False
        raise KeyError(rank)

    def __iter__(self):
        return iter(list(self._index) + self._absent)

    def __len__(self) -> int:
        return len(self._index) + len(self._absent)


class BwdResult(NamedTuple):
    dq: torch.Tensor
    dk_by_owner: Dict[int, torch.Tensor]
    dv_by_owner: Dict[int, torch.Tensor]
    attended: OwnerFlags
    dk: torch.Tensor
    dv: torch.Tensor


def _check_qkv(q, k, v, seg: Segments):
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k, v)), "q, k, v must be contiguous device tensors")
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "dtype must be bfloat16 or float32")
    _need(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "q [B,Hq,L,D], k/v [B,Hkv,S,D]")
    B, Hq, L, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    _need(B == Bk == seg.B and L == seg.L and S == seg.S and D == Dk,
          f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} segments B={seg.B} L={seg.L} S={seg.S}")
    return B, Hq, Hkv, L, S, D


def attn_fwd(q: torch.Tensor, k_nb: torch.Tensor, v_nb: torch.Tensor, seg: Segments,
             scale: Optional[float] = None, dropout_p: float = 0.0):
    """Forward; returns ``(out [B,Hq,L,D], saved)``.  ``scale=None`` means ``D ** -0.5``."""
    lib = _lib.load()
    B, Hq, Hkv, L, S, D = _check_qkv(q, k_nb, v_nb, seg)
    scale = D ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q)
    resid = torch.empty(q.shape, dtype=torch.int8, device=q.device) if q.dtype == torch.bfloat16 else None
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    _lib.check(lib.nb_attn_fwd(_ptr(q), _ptr(k_nb), _ptr(v_nb), _ptr(out), _ptr(resid), _ptr(lse), _ptr(seg.buf),
                               B, Hq, Hkv, L, S, D, scale, seg.window, float(dropout_p), _DTYPES[q.dtype],
                               None, 0, _stream_ptr(q.device)), "nb_attn_fwd")
    return out, Saved(q, k_nb, v_nb, out, resid, lse, seg, scale)


def attn_bwd(saved: Saved, grad_out: torch.Tensor, owners: Optional[OwnerTable] = None,
             stored_ds: bool = True) -> BwdResult:
    """Backward from the saved forward (no recompute).  ``stored_ds``: with a
    left window, give the library room to store dS and form dQ from it (the
    faster form; dK/dV identical, dQ equal up to rounding order); ``False``
    keeps the dQ pass that recomputes S and dP.

    Returns ``BwdResult(dq, dk_by_owner, dv_by_owner, attended, dk, dv)``; the
    per-owner entries are views of ``dk``/``dv`` (exact zeros for owners that were
    not attended) plus zero tensors for owners outside the neighbourhood.
    """
    lib = _lib.load()
    q, k, v, out, resid, lse, seg, scale = saved
    B, Hq, Hkv, L, S, D = _check_qkv(q, k, v, seg)
    _need(grad_out.shape == q.shape and grad_out.dtype == q.dtype and grad_out.is_contiguous(),
          "grad_out must match q")
    owners = OwnerTable.single(S) if owners is None else owners
    off = [int(x) for x in owners.offsets]
    n_owner = len(off) - 1
    _need(n_owner == len(owners.owners), "offsets must have len(owners) + 1 entries")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    att = torch.empty((max(n_owner, 1),), dtype=torch.uint8, device=q.device)
    # with a window, room for the banded dS (the backward then forms dQ from it)
    ws_bytes = (lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S, D, _DTYPES[q.dtype], seg.window)
                if stored_ds else lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, _DTYPES[q.dtype]))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    off_c = (ctypes.c_int32 * len(off))(*off)
    _lib.check(lib.nb_attn_bwd(_ptr(grad_out), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(resid), _ptr(lse),
                               _ptr(seg.buf),
                               _ptr(seg.folded), B, Hq, Hkv, L, S, D, scale, seg.window, _DTYPES[q.dtype],
                               _ptr(dq), _ptr(dk), _ptr(dv), ctypes.cast(off_c, ctypes.c_void_p), n_owner,
                               _ptr(att), _ptr(ws), ws_bytes, _stream_ptr(q.device)), "nb_attn_bwd")
    dk_by, dv_by, absent = {}, {}, []
    for o, rank in enumerate(owners.owners):
        dk_by[rank] = dk[:, :, off[o]:off[o + 1]]
        dv_by[rank] = dv[:, :, off[o]:off[o + 1]]
    n_prior = owners.n_prior if owners.n_prior is not None else len(owners.owners) - 1
    for d in range(n_prior + 1):
        r = (owners.cp_rank - d) % owners.cp_size
        if r not in dk_by:
            shape = (B, Hkv, L, D)  # a ring owner's chunk is one shard long
            dk_by[r] = torch.zeros(shape, dtype=k.dtype, device=k.device)
            dv_by[r] = torch.zeros(shape, dtype=v.dtype, device=v.device)
            absent.append(r)
    return BwdResult(dq, dk_by, dv_by, OwnerFlags(att[:n_owner], list(owners.owners), absent), dk, dv)


class NeighbourhoodAttention(torch.autograd.Function):
    """Autograd wrapper: forward saves (O, LSE), backward runs the library backward."""

    @staticmethod
    def forward(ctx, q, k, v, seg: Segments, scale: Optional[float] = None):
        out, saved = attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), seg, scale)
        ctx.saved_meta = (seg, saved.scale, saved.out_resid is not None)
        ctx.save_for_backward(saved.q, saved.k, saved.v, saved.out,
                              saved.out_resid if saved.out_resid is not None else saved.lse, saved.lse)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        q, k, v, out, resid, lse = ctx.saved_tensors
        seg, scale, has_resid = ctx.saved_meta
        r = attn_bwd(Saved(q, k, v, out, resid if has_resid else None, lse, seg, scale), grad_out.contiguous())
        return r.dq, r.dk, r.dv, None, None


def neighbourhood_attention(q, k, v, seg: Segments, scale: Optional[float] = None):
    return NeighbourhoodAttention.apply(q, k, v, seg, scale)


# ------------------------------------------------------------------ zero-copy neighbourhood
@dataclass
class KvChunk:
    """One owner chunk of the neighbourhood, used in place: keys are rows
    ``[start, start + length)`` of ``k`` / ``v`` ``[B, Hkv, rows, D]``."""

    k: torch.Tensor
    v: torch.Tensor
    start: int
    length: int


class ChunkSaved(NamedTuple):
    q: torch.Tensor
    chunks: List[KvChunk]
    out: torch.Tensor
    out_resid: Optional[torch.Tensor]
    lse: torch.Tensor
    seg: Segments
    scale: float


def ring_window_chunks(k_chunks: List[torch.Tensor], v_chunks: List[torch.Tensor], window: int) -> List[KvChunk]:
    """The windowed ring neighbourhood without a copy: of the causally valid chunks
    ``0..cp_rank`` (each ``[B, Hkv, L, D]``, the last one the rank's own), keep the
    own chunk and the last ``window`` keys before it -- the only keys a left window
    of ``window`` reaches from the shard (cp_local_ring page, module docstring)."""
    _need(len(k_chunks) == len(v_chunks) and k_chunks, "one K and one V buffer per chunk")
    L = k_chunks[-1].shape[2]
    need = L * (len(k_chunks) - 1) if window is None or window < 0 else min(int(window), L * (len(k_chunks) - 1))
    out: List[KvChunk] = []
    left = need
    for kc, vc in zip(reversed(k_chunks[:-1]), reversed(v_chunks[:-1])):
        if left <= 0:
            break
        n = min(left, kc.shape[2])
        out.append(KvChunk(kc, vc, kc.shape[2] - n, n))
        left -= n
    out.reverse()
    out.append(KvChunk(k_chunks[-1], v_chunks[-1], 0, L))
    return out


def _chunk_args(chunks: List[KvChunk], q: torch.Tensor, seg: Segments):
    _need(1 <= len(chunks) <= 16, "1 to 16 chunks")
    B, Hq, L, D = q.shape
    for c in chunks:
        _need(c.k.is_cuda and c.k.is_contiguous() and c.v.is_contiguous() and c.k.shape == c.v.shape
              and c.k.dtype == q.dtype and c.v.dtype == q.dtype and c.k.dim() == 4, "chunk buffers [B, Hkv, rows, D]")
        _need(c.k.shape[0] == B and c.k.shape[3] == D and c.k.shape[1] == chunks[0].k.shape[1], "chunk shapes")
        _need(0 <= c.start and c.length >= 1 and c.start + c.length <= c.k.shape[2], "chunk row range")
    S = sum(c.length for c in chunks)
    _need(S == seg.S and L == seg.L and B == seg.B, "the chunks must cover the segments' neighbourhood")
    n = len(chunks)
    P = ctypes.c_void_p * n
    I = ctypes.c_int32 * n
    return (B, Hq, chunks[0].k.shape[1], L, S, D, n,
            P(*[c.k.data_ptr() for c in chunks]), P(*[c.v.data_ptr() for c in chunks]),
            I(*[c.length for c in chunks]), I(*[c.start for c in chunks]), I(*[c.k.shape[2] for c in chunks]))


def attn_fwd_chunks(q: torch.Tensor, chunks: List[KvChunk], seg: Segments, scale: Optional[float] = None):
    """Forward reading K/V in place from the chunk buffers; returns ``(out, saved)``."""
    lib = _lib.load()
    _need(q.is_cuda and q.is_contiguous() and q.dtype in _DTYPES and q.dim() == 4, "q [B,Hq,L,D] on the device")
    B, Hq, Hkv, L, S, D, n, kp, vp, ln, st, rw = _chunk_args(chunks, q, seg)
    scale = D ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q)
    resid = torch.empty(q.shape, dtype=torch.int8, device=q.device) if q.dtype == torch.bfloat16 else None
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    _lib.check(lib.nb_attn_fwd_chunks(_ptr(q), ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
                                      ctypes.cast(ln, ctypes.c_void_p), ctypes.cast(st, ctypes.c_void_p),
                                      ctypes.cast(rw, ctypes.c_void_p), n, _ptr(out), _ptr(resid), _ptr(lse),
                                      _ptr(seg.buf), B, Hq, Hkv, L, S, D, scale, seg.window, 0.0, _DTYPES[q.dtype],
                                      None, 0, _stream_ptr(q.device)), "nb_attn_fwd_chunks")
    return out, ChunkSaved(q, list(chunks), out, resid, lse, seg, scale)


def attn_bwd_chunks(saved: ChunkSaved, grad_out: torch.Tensor, stored_ds: bool = True):
    """Backward writing whole chunk-gradient buffers (zeros outside the used rows
    and for keys no query attends); returns ``(dq, [dk_c], [dv_c], attended)``
    where ``attended`` is an :class:`OwnerFlags` keyed by chunk index (read
    lazily: the call itself never synchronises).  ``stored_ds`` as for
    :func:`attn_bwd`."""
    lib = _lib.load()
    q, chunks, out, resid, lse, seg, scale = saved
    _need(grad_out.shape == q.shape and grad_out.dtype == q.dtype and grad_out.is_contiguous(),
          "grad_out must match q")
    B, Hq, Hkv, L, S, D, n, kp, vp, ln, st, rw = _chunk_args(chunks, q, seg)
    dq = torch.empty_like(q)
    dks = [torch.empty_like(c.k) for c in chunks]
    dvs = [torch.empty_like(c.v) for c in chunks]
    att = torch.empty((n,), dtype=torch.uint8, device=q.device)
    ws_bytes = (lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S, D, _DTYPES[q.dtype], seg.window)
                if stored_ds else lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, _DTYPES[q.dtype]))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    P = ctypes.c_void_p * n
    dkp, dvp = P(*[t.data_ptr() for t in dks]), P(*[t.data_ptr() for t in dvs])
    _lib.check(lib.nb_attn_bwd_chunks(_ptr(grad_out), _ptr(q), ctypes.cast(kp, ctypes.c_void_p),
                                      ctypes.cast(vp, ctypes.c_void_p), ctypes.cast(ln, ctypes.c_void_p),
                                      ctypes.cast(st, ctypes.c_void_p), ctypes.cast(rw, ctypes.c_void_p), n,
                                      _ptr(out), _ptr(resid), _ptr(lse), _ptr(seg.buf), _ptr(seg.folded), B, Hq, Hkv,
                                      L, S, D, scale, seg.window, _DTYPES[q.dtype], _ptr(dq),
                                      ctypes.cast(dkp, ctypes.c_void_p), ctypes.cast(dvp, ctypes.c_void_p), _ptr(att),
                                      _ptr(ws), ws_bytes, _stream_ptr(q.device)), "nb_attn_bwd_chunks")
    return dq, dks, dvs, OwnerFlags(att, list(range(n)), [])

