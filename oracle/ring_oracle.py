"""fp64 CPU oracle for the global-layer ring attention of one context-parallel
rank: per-chunk attention with an online-softmax merge.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, and by nothing else; it shares no code with the
HIP library and never imports it.  Written to be read against the NeMo
AutoModel ``gemma4_moe.cp_attention`` page:

* ``_run_gemma4_cp_ffpa_varlen_ring_forward``: rank r's queries (its own chunk
  of the global sequence) visit the K/V chunks of owners r, r-1, ..., 0 (chunks
  of later owners are causally skipped); each chunk's attention gives an
  ``(out, lse)`` pair, merged into fp32 running accumulators; padding query
  rows stay 0.
* ``_chunk_dense_eligible`` and ``_build_packed_ring_segments``: the own chunk
  runs causally, an earlier owner's chunk non-causally (every one of its keys
  precedes every query); in both, a query only meets keys of its own document
  (the per-document segments pair a document's query tokens with its key
  tokens; id 0 is padding).
* ``_merge_flex_chunk`` / ``_merge_ffpa_packed_chunk``: the online-softmax
  merge of two partial results; the ``-inf``-safe form keeps a row that
  neither side covered at 0 (its lse stays ``-inf``) instead of NaN.
* ``_merge_live_chunk_``: the same merge applied in place at a given set of
  rows only.
* ``_ffpa_varlen_backward_chunk``: each chunk's backward uses the *global*
  merged out and lse; the chunks' dQ add up, and each chunk's dK/dV is its
  owner's contribution (``_route_kv_grads_to_owners`` sums them per owner).

Readings where the page is silent: positions are global (query row i of rank r
sits at ``r Lc + i``, key j of owner o at ``o Lc + j``); LSE is the natural
log of the softmax denominator; the GQA head map is ``kv = h // (Hq // Hkv)``;
a chunk that leaves a query row without keys gives that row ``out = 0``,
``lse = -inf``.  The merge is written with its two explicit weights
``exp(lse_x - lse_new)`` (the page's single lerp is the same combination, the
weights summing to one).
"""
from __future__ import annotations

import numpy as np

__all__ = ["chunk_mask", "chunk_forward", "merge", "merge_live", "chunk_backward", "ring_forward",
           "ring_backward"]


def _f64(x):
    if hasattr(x, "detach"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def chunk_mask(q_ids, k_ids, q_start, k_start, causal):
    """``[B, Lq, Lk]`` allow-mask of one (query shard, key chunk) pair: same
    document id > 0 on both sides and, when causal, the key's global position
    ``k_start + j`` not after the query's ``q_start + i``."""
    q_ids = np.asarray(q_ids)
    k_ids = np.asarray(k_ids)
    M = (q_ids[:, :, None] == k_ids[:, None, :]) & (q_ids[:, :, None] > 0)
    if causal:
        qp = q_start + np.arange(q_ids.shape[1])
        kp = k_start + np.arange(k_ids.shape[1])
        M &= kp[None, None, :] <= qp[None, :, None]
    return M


def chunk_forward(q, k, v, q_ids, k_ids, q_start, k_start, causal, scale):
    """One key chunk's attention: ``(out [B, Hq, Lq, D], lse [B, Hq, Lq])``,
    the softmax over the chunk's allowed keys only (``_ffpa_varlen_forward_chunk``)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, D = q.shape
    grp = Hq // k.shape[1]
    M = chunk_mask(q_ids, k_ids, q_start, k_start, causal)
    out = np.zeros((B, Hq, Lq, D))
    lse = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        rows = M[b].any(axis=1)
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // grp].T)
            s = np.where(M[b], s, -np.inf)
            m = np.where(rows, s.max(axis=1), 0.0)
            e = np.where(M[b], np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            out[b, h][rows] = (e[rows] @ v[b, h // grp]) / den[rows, None]
            lse[b, h][rows] = m[rows] + np.log(den[rows])
    return out, lse


def merge(out_acc, lse_acc, out_step, lse_step):
    """Online-softmax merge of two partial results over disjoint key sets
    (``_merge_ffpa_packed_chunk``): ``lse = log(e^lse_acc + e^lse_step)``, out the
    two outs weighted by ``exp(lse_x - lse)``; a row with both lse ``-inf``
    keeps out 0 and lse ``-inf``.  ``out_acc=None`` (nothing merged yet) returns
    the step."""
    out_step, lse_step = _f64(out_step), _f64(lse_step)
    if out_acc is None:
        return out_step.copy(), lse_step.copy()
    out_acc, lse_acc = _f64(out_acc), _f64(lse_acc)
    hi = np.maximum(lse_acc, lse_step)
    live = np.isfinite(hi)
    hs = np.where(live, hi, 0.0)
    den = np.where(live, np.exp(lse_acc - hs) + np.exp(lse_step - hs), 1.0)   # >= 1 on live rows
    lse = np.where(live, hs + np.log(den), -np.inf)
    w_acc = np.where(live, np.exp(lse_acc - np.where(live, lse, 0.0)), 0.0)
    w_step = np.where(live, np.exp(lse_step - np.where(live, lse, 0.0)), 0.0)
    out = w_acc[..., None] * out_acc + w_step[..., None] * out_step
    return out, lse


def merge_live(out_acc, lse_acc, out_step, lse_step, flat_index):
    """``_merge_live_chunk_``: merge in place at the rows ``flat_index`` (indices
    ``b * S + s`` into the ``[B, S]`` row grid, every head) and leave every other
    row as it is.  Returns new arrays."""
    out_acc, lse_acc = _f64(out_acc).copy(), _f64(lse_acc).copy()
    out_step, lse_step = _f64(out_step), _f64(lse_step)
    B, H, S, D = out_acc.shape
    idx = np.asarray(flat_index, dtype=np.int64)
    b, s = idx // S, idx % S
    o, l = merge(out_acc[b, :, s], lse_acc[b, :, s], out_step[b, :, s], lse_step[b, :, s])
    out_acc[b, :, s] = o
    lse_acc[b, :, s] = l
    return out_acc, lse_acc


def chunk_backward(q, k, v, dout, out, lse, q_ids, k_ids, q_start, k_start, causal, scale):
    """One chunk's backward with the *global* out and lse
    (``_ffpa_varlen_backward_chunk``): the probabilities ``exp(scale q.k - lse)``
    of the chunk's allowed keys, ``Delta = rowsum(dout * out)`` over the global
    out, ``dS = P (dP - Delta)``; returns the chunk's contributions
    ``(dQ [B, Hq, Lq, D], dK, dV [B, Hkv, Lk, D])``."""
    q, k, v, dout, out, lse = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(out), _f64(lse)
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    M = chunk_mask(q_ids, k_ids, q_start, k_start, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = h // grp
            l = lse[b, h]
            fin = np.isfinite(l)
            s = scale * (q[b, h] @ k[b, kv].T)
            P = np.where(M[b] & fin[:, None], np.exp(s - np.where(fin, l, 0.0)[:, None]), 0.0)
            dP = dout[b, h] @ v[b, kv].T
            delta = (dout[b, h] * out[b, h]).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dq[b, h] = scale * (dS @ k[b, kv])
            dk[b, kv] += scale * (dS.T @ q[b, h])
            dv[b, kv] += P.T @ dout[b, h]
    return dq, dk, dv


def ring_forward(q, k_chunks, v_chunks, ids, rank, scale):
    """Rank ``rank``'s ring forward: ``q`` ``[B, Hq, Lc, D]`` is its chunk's
    queries, ``k_chunks[o]`` / ``v_chunks[o]`` ``[B, Hkv, Lc, D]`` owner o's keys
    (o = 0 .. rank), ``ids`` ``[B, N]`` the folded global doc map.  Visits the
    own chunk (causal) first, then owners rank-1, ..., 0 (non-causal), merging
    each; returns ``(out, lse)``."""
    Lc = _f64(q).shape[2]
    q_start = rank * Lc
    q_ids = np.asarray(ids)[:, q_start:q_start + Lc]
    out = lse = None
    for o in range(rank, -1, -1):
        k_ids = np.asarray(ids)[:, o * Lc:(o + 1) * Lc]
        so, sl = chunk_forward(q, k_chunks[o], v_chunks[o], q_ids, k_ids, q_start, o * Lc, o == rank, scale)
        out, lse = merge(out, lse, so, sl)
    return out, lse


def ring_backward(q, k_chunks, v_chunks, dout, out, lse, ids, rank, scale):
    """Every chunk's backward with the global out/lse: ``(dQ, [dK_o], [dV_o])``,
    dQ the sum of the chunks' contributions."""
    Lc = _f64(q).shape[2]
    q_start = rank * Lc
    q_ids = np.asarray(ids)[:, q_start:q_start + Lc]
    dq = np.zeros(_f64(q).shape)
    dks, dvs = [], []
    for o in range(rank + 1):
        k_ids = np.asarray(ids)[:, o * Lc:(o + 1) * Lc]
        a, bk, bv = chunk_backward(q, k_chunks[o], v_chunks[o], dout, out, lse, q_ids, k_ids, q_start, o * Lc,
                                   o == rank, scale)
        dq += a
        dks.append(bk)
        dvs.append(bv)
    return dq, dks, dvs
