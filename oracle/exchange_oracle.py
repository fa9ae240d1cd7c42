"""CPU oracle for the block-diagonal context-parallel K/V exchange plans and for
the needed-range exchange, emulated for every rank on one device.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests and by the
benchmark's CPU-baseline leg, and by nothing else.  It shares no code with the
HIP library and never imports it.  It follows the NeMo AutoModel
``blockdiag_cp.exchange`` page:

* the global left-halo plan (its description): every rank ``r`` of a world of
  ``cp`` ranks owns the chunk ``[r L, (r + 1) L)`` of the global sequence and
  needs the contiguous K/V range ``[s_first_r, real_end_r)`` -- the part of its
  boundary document that earlier ranks own (the straddle) plus its own chunk.
  ``back_r = r L - s_first_r`` is the straddle length; a single neighbour
  exchange suffices (``use_halo``) iff ``back_r <= L`` for every rank.  All
  ranks derive the plan from the same replicated document ids.
* ``_LeftHaloExchange``: one uniform-size exchange; each rank receives the
  last ``halo_size`` tokens of the previous rank's chunk and keeps the last
  ``back_r`` of them.
* the per-(source, destination) split description and ``_NeededKVExchange``:
  source ``s`` sends destination ``r`` the intersection of its chunk with
  ``r``'s needed range (a token goes once to every rank that needs it; the send
  buffer is the local chunk gathered through ``send_index``); the receiver
  concatenates the pieces in source order into its contiguous needed range.
  The backward adds every destination's gradient back onto the source token
  (index_add).

Readings where the page is silent (also listed in the design notes):
* padding (nonzero pad mask) is folded to document id 0 first; id 0 is never a
  document;
* ``s_first_r`` is the start of the run of equal nonzero ids that holds
  position ``r L``; ``r L`` itself when that position is padding;
* ``real_end_r`` is one past the last non-padding position of chunk ``r``; a
  chunk without one needs nothing (``s_first_r = real_end_r = r L``);
* with several batch rows the range is the union over the rows (one range per
  rank serves the whole ``[B, C, L, D]`` chunk);
* ``back_r = r L - s_first_r``; ``halo_size = max_r back_r``.
"""
from __future__ import annotations

import numpy as np

__all__ = ["needed_ranges", "halo_plan", "a2a_plan", "a2a_forward", "a2a_backward"]


def _folded(doc_ids, pad_mask):
    ids = np.array(doc_ids, dtype=np.int64, copy=True)
    if ids.ndim == 1:
        ids = ids[None, :]
    if pad_mask is not None:
        pm = np.asarray(pad_mask)
        if pm.ndim == 1:
            pm = pm[None, :]
        ids[pm != 0] = 0
    ids[ids < 0] = 0
    return ids


def needed_ranges(doc_ids, pad_mask, cp_size):
    """Per rank ``(s_first, real_end)`` of the needed K/V range (global positions).

    ``doc_ids`` is ``[B, N]`` (or ``[N]``) with ``N = cp_size * L``.
    """
    ids = _folded(doc_ids, pad_mask)
    B, N = ids.shape
    if N % cp_size:
        raise ValueError("the sequence must split into cp_size equal chunks")
    L = N // cp_size
    s_first = np.zeros(cp_size, dtype=np.int64)
    real_end = np.zeros(cp_size, dtype=np.int64)
    for r in range(cp_size):
        lo, hi = r * L, (r + 1) * L
        firsts, ends = [], []
        for b in range(B):
            row = ids[b]
            real = np.nonzero(row[lo:hi] != 0)[0]
            if real.size == 0:
                continue                       # this row needs nothing from rank r's view
            ends.append(lo + int(real[-1]) + 1)
            if row[lo] == 0:
                firsts.append(lo)
                continue
            j = lo                             # walk back to the start of the run holding lo
            while j > 0 and row[j - 1] == row[lo]:
                j -= 1
            firsts.append(j)
        if ends:
            s_first[r], real_end[r] = min(firsts), max(ends)
        else:
            s_first[r] = real_end[r] = lo
    return s_first, real_end


def halo_plan(doc_ids, pad_mask, cp_size):
    """The left-halo plan: ranges, straddle lengths, ``use_halo``, ``halo_size``."""
    ids = _folded(doc_ids, pad_mask)
    L = ids.shape[1] // cp_size
    s_first, real_end = needed_ranges(doc_ids, pad_mask, cp_size)
    back = np.array([r * L - s_first[r] for r in range(cp_size)], dtype=np.int64)
    return {
        "L": L,
        "s_first": s_first,
        "real_end": real_end,
        "back": back,
        "use_halo": bool(np.all(back <= L)),
        "halo_size": int(back.max()) if cp_size else 0,
    }


def a2a_plan(doc_ids, pad_mask, cp_size):
    """The needed-only all-to-all-v plan.

    Returns the halo-plan fields plus ``splits[s, r]`` (tokens source ``s`` sends
    destination ``r``; ``in_splits`` of ``s`` is row ``s``, ``out_splits`` of
    ``r`` is column ``r``) and ``send_index[s]`` (local indices into chunk ``s``,
    the pieces for destinations 0, 1, ... one after another).
    """
    plan = halo_plan(doc_ids, pad_mask, cp_size)
    L, s_first, real_end = plan["L"], plan["s_first"], plan["real_end"]
    splits = np.zeros((cp_size, cp_size), dtype=np.int64)
    send_index = []
    for s in range(cp_size):
        own = np.arange(s * L, (s + 1) * L)
        idx = []
        for r in range(cp_size):
            piece = own[(own >= s_first[r]) & (own < real_end[r])]
            splits[s, r] = piece.size
            idx.extend((piece - s * L).tolist())
        send_index.append(np.array(idx, dtype=np.int64))
    plan["splits"] = splits
    plan["send_index"] = send_index
    return plan


def a2a_forward(x, plan):
    """Every rank's received needed range: ``x`` is the global ``[B, C, N, D]``
    tensor (rank ``s`` owns ``x[:, :, s L:(s + 1) L]``).  Source ``s`` gathers
    its send buffer through ``send_index``, cuts it by its ``in_splits``, and
    each destination concatenates its pieces in source order."""
    x = np.asarray(x, dtype=np.float64)
    cp, L = len(plan["send_index"]), plan["L"]
    splits = plan["splits"]
    pieces = [[None] * cp for _ in range(cp)]     # pieces[s][r]
    for s in range(cp):
        send = x[:, :, s * L + plan["send_index"][s], :]
        off = 0
        for r in range(cp):
            pieces[s][r] = send[:, :, off:off + splits[s, r], :]
            off += splits[s, r]
    return [np.concatenate([pieces[s][r] for s in range(cp)], axis=2) for r in range(cp)]


def a2a_backward(grads, plan, shape):
    """The exchange's backward: ``grads[r]`` is the gradient of rank ``r``'s
    received range.  Each destination hands every source its piece back; the
    source adds it onto its chunk at ``send_index`` (index_add).  Returns the
    global ``[B, C, N, D]`` gradient (zero where no rank needed a token)."""
    cp, L = len(plan["send_index"]), plan["L"]
    splits = plan["splits"]
    out = np.zeros(shape, dtype=np.float64)
    for s in range(cp):
        back = []
        for r in range(cp):
            g = np.asarray(grads[r], dtype=np.float64)
            off = int(splits[:s, r].sum())         # source s's piece inside r's range
            back.append(g[:, :, off:off + splits[s, r], :])
        recv = np.concatenate(back, axis=2)        # in the order of the send buffer
        np.add.at(out, (slice(None), slice(None), s * L + plan["send_index"][s]), recv)
    return out
