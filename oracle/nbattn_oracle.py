"""fp64 CPU oracle for one context-parallel rank's neighbourhood attention.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg, and by nothing else.  It shares
no code with the HIP library (no kernels, headers, helpers or tables) and never
imports it.  It is written to be read against the pages it follows:

* NeMo AutoModel ``blockdiag_cp.kernels`` page, ``_cp_blockdiag_mask``: the
  dense boolean allow-mask ``[B, 1, L, S]`` -- a query may attend a key iff both
  carry the same document id, neither is padding (id 0), and the key's position
  is not after the query's; the diagonal is always allowed.
* the same page, ``_cp_blockdiag_varlen``: the varlen computation equals that
  mask followed by scaled-dot-product attention on the real (non-padding)
  query rows; padding query rows are zeros.
* NeMo AutoModel ``cp_local_ring`` page, module docstring: the local query shard
  is the suffix of the concatenated neighbourhood, so one bottom-right-aligned
  causal call with a *left window* covers it.  The window follows
  FlashAttention's ``window_size[0]`` convention: a key ``j`` is inside the
  window of query position ``p`` iff ``p - j <= W`` (``W < 0``: no window).
* the same page, ``_fold_pad``: padding is folded into the doc map as id 0.
* the same page, ``_owner_grad_dict``: dK/dV are handed back per owner chunk,
  with zeros for chunks the shard did not attend.
* the same page, ``sliding_ring_compute_fa_fwd`` / ``_bwd``: the forward keeps
  what the backward needs (output and log-sum-exp), the backward returns
  ``(dQ, dK by owner, dV by owner)``.

Readings where the pages are silent (stated once here, applied throughout):
LSE is the natural log of the softmax denominator, fp64 here; the GQA head
map is ``kv = h // (Hq // Hkv)``; a padding mask is nonzero at padding;
document ids <= 0 are treated like padding (only ids > 0 are documents);
padding query rows get ``O = 0``, ``LSE = -inf``, ``dQ = 0`` and contribute
nothing to dK/dV.

Every function computes on float64 copies of the exact input values.  Row
blocks only bound memory; they do not change the arithmetic of a row.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "fold_pad", "allow_mask", "real_rows", "attention_forward", "attention_backward",
    "key_attended", "owner_split", "segments_reference", "useful_pairs",
]


def _f64(x):
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any float dtype."""
    if hasattr(x, "detach"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def fold_pad(doc_ids, pad_mask=None):
    """``cp_local_ring`` page, ``_fold_pad``: padding positions become doc id 0.

    ``doc_ids`` is ``[B, S]`` (ints), ``pad_mask`` ``[B, S]`` with nonzero at
    padding, or ``None`` (ids returned unchanged).
    """
    ids = np.asarray(doc_ids).astype(np.int64)
    if pad_mask is None:
        return ids.copy()
    return np.where(np.asarray(pad_mask) != 0, 0, ids)


def allow_mask(folded, L, window, rows=None):
    """``blockdiag_cp.kernels`` page, ``_cp_blockdiag_mask``, plus the left window.

    ``folded`` is the folded doc map ``[B, S]`` of the neighbourhood; local query
    row ``i`` sits at neighbourhood position ``p = S - L + i`` (bottom-right
    alignment).  Returns a boolean ``[B, 1, R, S]`` for the rows ``rows``
    (default: all ``L``): ``M = (same doc & doc > 0 & j <= p & window) | (j == p)``.
    """
    folded = np.asarray(folded)
    B, S = folded.shape
    i = np.arange(L) if rows is None else np.asarray(rows)
    p = S - L + i
    j = np.arange(S)
    idp = folded[:, p]
    same_doc = (idp[:, :, None] == folded[:, None, :]) & (idp[:, :, None] > 0)
    causal = j[None, :] <= p[:, None]
    m = same_doc & causal[None, :, :]
    if window is not None and window >= 0:
        m &= ((p[:, None] - j[None, :]) <= window)[None, :, :]
    m |= (j[None, :] == p[:, None])[None, :, :]
    return m[:, None, :, :]


def real_rows(folded, L):
    """Query rows whose position carries a document (``_cp_blockdiag_varlen``: real rows)."""
    folded = np.asarray(folded)
    S = folded.shape[1]
    return folded[:, S - L:] > 0


def _row_blocks(rows, block):
    for s in range(0, len(rows), block):
        yield rows[s:s + block]


def _probs(q_rows, k_b, M, real, scale):
    """Softmax probabilities of one row block: ``P = exp(s - LSE)`` on the mask, 0 elsewhere.

    Returns ``(P, LSE)``; padding rows get ``P = 0`` and ``LSE = -inf``.
    """
    s = scale * (q_rows @ k_b.T)
    s = np.where(M, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)          # finite: every row has its diagonal
    e = np.exp(s - mx)
    z = e.sum(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(z[:, 0])
    p = e / z
    p[~real] = 0.0
    lse = np.where(real, lse, -np.inf)
    return p, lse


def attention_forward(q, k, v, folded, window, scale, heads=None, rows=None, row_block=256):
    """Forward of ``sliding_ring_compute_fa_fwd`` / ``_cp_blockdiag_varlen`` by definition.

    ``q`` ``[B, Hq, L, D]``, ``k``/``v`` ``[B, Hkv, S, D]`` (any float dtype, taken
    exactly in fp64).  ``heads``: q heads to compute (default all); ``rows``: local
    query rows to compute (default all).  Returns ``(O, LSE)`` with shapes
    ``[B, len(heads), len(rows), D]`` and ``[B, len(heads), len(rows)]``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    folded = np.asarray(folded)
    B, Hq, L, D = q.shape
    g = Hq // k.shape[1]
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.arange(L) if rows is None else np.asarray(rows)
    O = np.zeros((B, len(heads), len(rows), D))
    LSE = np.full((B, len(heads), len(rows)), -np.inf)
    for b in range(B):
        real_b = real_rows(folded[b:b + 1], L)[0]
        for hi, h in enumerate(heads):
            kv = h // g
            for s0 in range(0, len(rows), row_block):
                blk = rows[s0:s0 + row_block]
                M = allow_mask(folded[b:b + 1], L, window, rows=blk)[0, 0]
                P, lse = _probs(q[b, h, blk], k[b, kv], M, real_b[blk], scale)
                O[b, hi, s0:s0 + len(blk)] = P @ v[b, kv]
                LSE[b, hi, s0:s0 + len(blk)] = lse
    return O, LSE


def attention_backward(q, k, v, dout, folded, window, scale, kv_heads=None, rows=None, keys=None,
                       row_block=256):
    """Analytic gradients of ``sum(O * dO)`` (``sliding_ring_compute_fa_bwd`` by definition).

    With ``P`` the softmax probabilities above:
    ``dP = dO V^T``, ``Delta_i = sum_j P_ij dP_ij``, ``dS = P * (dP - Delta)``,
    ``dQ = scale dS K``, ``dK = scale sum_{h in group} dS^T Q_h``,
    ``dV = sum_{h in group} P^T dO_h``.  Padding rows contribute nothing and get
    ``dQ = 0``.  ``kv_heads``: kv heads (and their q-head groups) to compute.
    ``rows``: only these local query rows enter the sums (dQ of other rows is
    left 0; dK/dV are then exact at every key no other real row attends).
    ``keys``: dK/dV are accumulated only at these keys (others left 0).
    Returns ``(dQ [B,Hq,L,D], dK [B,Hkv,S,D], dV [B,Hkv,S,D])``; heads outside
    ``kv_heads`` are left zero.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    folded = np.asarray(folded)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    g = Hq // Hkv
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    rows = np.arange(L) if rows is None else np.asarray(rows)
    keys = np.arange(S) if keys is None else np.asarray(keys)
    for b in range(B):
        real_b = real_rows(folded[b:b + 1], L)[0]
        for kv in kv_heads:
            for h in range(kv * g, (kv + 1) * g):
                for blk in _row_blocks(rows, row_block):
                    M = allow_mask(folded[b:b + 1], L, window, rows=blk)[0, 0]
                    P, _ = _probs(q[b, h, blk], k[b, kv], M, real_b[blk], scale)
                    dP = dout[b, h, blk] @ v[b, kv].T
                    delta = (P * dP).sum(axis=1, keepdims=True)
                    dS = P * (dP - delta)
                    dQ[b, h, blk] = scale * (dS @ k[b, kv])
                    dK[b, kv, keys] += scale * (dS[:, keys].T @ q[b, h, blk])
                    dV[b, kv, keys] += P[:, keys].T @ dout[b, h, blk]
    return dQ, dK, dV


def key_attended(folded, L, window, row_block=512):
    """``[B, S]`` bool: key ``j`` is allowed for at least one real query row."""
    folded = np.asarray(folded)
    B, S = folded.shape
    out = np.zeros((B, S), dtype=bool)
    rows = np.arange(L)
    for b in range(B):
        real_b = real_rows(folded[b:b + 1], L)[0]
        for blk in _row_blocks(rows, row_block):
            M = allow_mask(folded[b:b + 1], L, window, rows=blk)[0, 0]
            out[b] |= M[real_b[blk]].any(axis=0)
    return out


def owner_split(dk, dv, owner_off, attended_keys):
    """``cp_local_ring`` page, ``_owner_grad_dict``: per-owner dK/dV chunks.

    ``owner_off`` are ascending neighbourhood offsets (``n_owner + 1`` entries).
    Returns ``(dk_list, dv_list, attended)`` where ``attended[o]`` says whether any
    real query attended a key of chunk ``o`` (``attended_keys`` from
    :func:`key_attended`).  Chunks that were not attended are exact zeros.
    """
    dk_l, dv_l, att = [], [], []
    for o in range(len(owner_off) - 1):
        a, e = owner_off[o], owner_off[o + 1]
        dk_l.append(dk[:, :, a:e])
        dv_l.append(dv[:, :, a:e])
        att.append(bool(np.asarray(attended_keys)[:, a:e].any()))
    return dk_l, dv_l, att


def segments_reference(folded, L, window):
    """Per-document varlen segments of the shard, by a plain loop over positions.

    Follows ``_cp_blockdiag_varlen`` (``blockdiag_cp.kernels`` page): every
    document the local rows touch becomes one segment whose query part is the
    local rows of that document and whose key part runs from the document's
    start to its last local row, so that bottom-right alignment reproduces the
    mask; and ``_cached_sliding_segments`` (``cp_local_ring`` page): with a
    window the key start of the straddling document is clipped at
    ``lo = max(0, S - L - W)``, which removes only keys no query can see.

    A document is a maximal run of one id > 0.  Segments are ordered by
    ``(b, position)``.  Returns a dict with ``n_seg``, ``cu_q``, ``cu_k``,
    ``q_row0`` (``b*L`` + first local row), ``k_row0`` (``b*S`` + first key),
    ``max_q``, ``max_k``, ``row_seg`` (segment of each local row, -1 for
    padding), ``row_klo`` (first key of the row's segment; ``p + 1`` for
    padding rows), ``kcov_lo`` (first covered key of each batch row, ``S`` if
    none), ``lo`` and ``status`` (bit 0: an id occurs in two separate runs of
    one row).
    """
    folded = np.asarray(folded)
    B, S = folded.shape
    lo = max(0, S - L - window) if (window is not None and window >= 0) else 0
    q0s, q1s, k0s, k1s, bs = [], [], [], [], []
    row_seg = np.full(B * L, -1, dtype=np.int64)
    row_klo = np.array([S - L + i + 1 for _ in range(B) for i in range(L)], dtype=np.int64)
    kcov_lo = np.full(B, S, dtype=np.int64)
    status = 0
    for b in range(B):
        runs = []
        j = 0
        while j < S:
            d = int(folded[b, j])
            if d > 0:
                a = j
                while j < S and int(folded[b, j]) == d:
                    j += 1
                runs.append((a, j, d))
            else:
                j += 1
        seen = set()
        for (_, _, d) in runs:
            if d in seen:
                status |= 1
            seen.add(d)
        for (a, e, d) in runs:
            if e <= S - L:
                continue
            sid = len(q0s)
            q0, q1 = max(a, S - L) - (S - L), e - (S - L)
            k0, k1 = max(a, lo), e
            q0s.append(q0), q1s.append(q1), k0s.append(k0), k1s.append(k1), bs.append(b)
            for i in range(q0, q1):
                row_seg[b * L + i] = sid
                row_klo[b * L + i] = k0
            if kcov_lo[b] == S:
                kcov_lo[b] = k0
    n = len(q0s)
    ql = np.array([q1s[s] - q0s[s] for s in range(n)], dtype=np.int64)
    kl = np.array([k1s[s] - k0s[s] for s in range(n)], dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(kl)]).astype(np.int64)
    return dict(
        n_seg=n, lo=lo, status=status,
        cu_q=cu_q, cu_k=cu_k,
        q_row0=np.array([bs[s] * L + q0s[s] for s in range(n)], dtype=np.int64),
        k_row0=np.array([bs[s] * S + k0s[s] for s in range(n)], dtype=np.int64),
        max_q=int(ql.max()) if n else 0, max_k=int(kl.max()) if n else 0,
        row_seg=row_seg, row_klo=row_klo, kcov_lo=kcov_lo,
    )


def useful_pairs(folded, L, window, row_block=512):
    """Number of allowed (query, key) pairs over real query rows, summed over the batch.

    This is the count the throughput figure is priced on (per query head).
    """
    folded = np.asarray(folded)
    B = folded.shape[0]
    total = 0
    rows = np.arange(L)
    for b in range(B):
        real_b = real_rows(folded[b:b + 1], L)[0]
        for blk in _row_blocks(rows, row_block):
            M = allow_mask(folded[b:b + 1], L, window, rows=blk)[0, 0]
            total += int(M[real_b[blk]].sum())
    return total
