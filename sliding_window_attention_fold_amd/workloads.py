"""Seeded synthetic workloads for neighbourhood attention.

This module only draws inputs: packed document maps, padding masks and the
Q/K/V/dO tensors, with the shapes of the five workloads below.  It holds none
of the attention arithmetic, so both the HIP path and the fp64 oracle can be
fed from it without sharing any of the method's code.

Every workload is one context-parallel rank's shard.  The query shard of
length ``L`` is the suffix of the key/value neighbourhood of length ``S``
(NeMo AutoModel ``cp_local_ring`` page, module docstring: the collected
chunks with owner <= cp_rank are concatenated in ascending order and the local
query shard is their suffix).

Recipe (identical for every consumer):

* doc maps: ``numpy.random.Generator(PCG64(1000 + cfg))``.  The global
  sequence is filled left to right; each draw is a document length, clipped to
  the workload's range, truncated at the end of the sequence; ids are 1, 2, 3,
  ... in order.  Padding is applied afterwards as a separate ``uint8`` mask
  (nonzero = pad) so that the fold of padding into the doc map is exercised;
  the ids under the mask stay nonzero.
* tensors: ``torch.Generator('cpu').manual_seed(1000 + cfg)``; ``randn`` in
  float32 in the order Q, K, V, dO; the outlier workload then draws
  ``rand(Q.shape) < 0.01`` and ``rand(K.shape) < 0.01`` and scales those
  entries by 8; finally a round-to-nearest-even cast to bfloat16 (the float32
  debug twin skips the cast).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_doc_map", "make_tensors", "small_variant"]


@dataclass(frozen=True)
class Workload:
    """One rank's neighbourhood-attention shard.

    ``owner_off`` are the neighbourhood offsets of the owner chunks (ascending
    owners ``owners``), ``cp_rank``/``cp_size`` the simulated ring position.
    """

    cfg: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int
    S_global: int          # length of the simulated global (all-rank) row
    q_start: int           # global offset of the local query shard
    window: int            # left window (FlashAttention window_size[0]); -1 = none
    doc_len: Tuple         # ("uniform", lo, hi) | ("geometric", p, lo, hi) | ("lognormal", mu, sigma, lo, hi) | ("single",)
    pad_tail: int          # pad positions at the end of each global row
    mode: str              # "ring" | "halo" | "needed"
    cp_rank: int
    cp_size: int
    outliers: bool = False
    per_row_docs: bool = False  # draw an independent doc map for every batch row

    @property
    def seed(self) -> int:
        return 1000 + self.cfg

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload(1, "tiny shard (2-chunk ring, rank 1)", B=1, Hq=2, Hkv=1, D=64, L=128,
                S_global=256, q_start=128, window=64, doc_len=("uniform", 20, 90), pad_tail=16,
                mode="ring", cp_rank=1, cp_size=2),
    2: Workload(2, "sliding layer, 4-way ring rank 3", B=1, Hq=16, Hkv=8, D=256, L=4096,
                S_global=16384, q_start=12288, window=1024,
                doc_len=("geometric", 1.0 / 2048.0, 64, 16384), pad_tail=0,
                mode="ring", cp_rank=3, cp_size=4),
    3: Workload(3, "block-diagonal halo, rank 1 of 2", B=1, Hq=32, Hkv=8, D=128, L=8192,
                S_global=16384, q_start=8192, window=-1,
                doc_len=("lognormal", 7.5, 1.0, 32, 8192), pad_tail=0,
                mode="halo", cp_rank=1, cp_size=2),
    4: Workload(4, "single long document, needed range, rank 7 of 8", B=1, Hq=32, Hkv=8, D=128,
                L=8192, S_global=65536, q_start=57344, window=-1, doc_len=("single",), pad_tail=0,
                mode="needed", cp_rank=7, cp_size=8),
    5: Workload(5, "many short docs + pad tail, batched", B=4, Hq=8, Hkv=2, D=128, L=4096,
                S_global=8192, q_start=4096, window=512, doc_len=("uniform", 16, 512),
                pad_tail=1228, mode="ring", cp_rank=1, cp_size=2, outliers=True,
                per_row_docs=True),
}


def get(cfg: int) -> Workload:
    return WORKLOADS[cfg]


def _fill_row(rng: np.random.Generator, n: int, spec: Tuple) -> np.ndarray:
    """Global doc-id row of length ``n``: lengths drawn left to right, ids 1, 2, ..."""
    row = np.zeros(n, dtype=np.int32)
    kind = spec[0]
    if kind == "single":
        row[:] = 1
        return row
    pos, doc = 0, 1
    while pos < n:
        if kind == "uniform":
            length = int(rng.integers(spec[1], spec[2] + 1))
        elif kind == "geometric":
            length = int(np.clip(rng.geometric(spec[1]), spec[2], spec[3]))
        elif kind == "lognormal":
            length = int(np.clip(np.rint(rng.lognormal(spec[1], spec[2])), spec[3], spec[4]))
        else:
            raise ValueError(f"unknown length law {kind!r}")
        end = min(n, pos + length)
        row[pos:end] = doc
        pos, doc = end, doc + 1
    return row


@dataclass
class DocMap:
    """Neighbourhood doc map of one workload (before the pad fold)."""

    doc_ids: np.ndarray            # [B, S] int32, ids under the pad mask left nonzero
    pad_mask: Optional[np.ndarray]  # [B, S] uint8 (nonzero = pad) or None
    nb_start: int                  # global offset of neighbourhood position 0
    S: int
    owner_off: List[int] = field(default_factory=list)  # neighbourhood offsets, len n_owner + 1
    owners: List[int] = field(default_factory=list)     # owner rank of each chunk (ascending)


def global_doc_map(w: Workload):
    """The whole sequence's doc ids ``[B, S_global]`` (int32) and pad mask (or None),
    as every context-parallel rank holds them (replicated)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    n_rows = w.B if w.per_row_docs else 1
    rows = [_fill_row(rng, w.S_global, w.doc_len) for _ in range(n_rows)]
    glob = np.stack(rows * (w.B if not w.per_row_docs else 1)).astype(np.int32)
    pad = None
    if w.pad_tail > 0:
        pad = np.zeros_like(glob, dtype=np.uint8)
        pad[:, w.S_global - w.pad_tail:] = 1
    return glob, pad


def make_doc_map(w: Workload) -> DocMap:
    glob, pad = global_doc_map(w)
    q_end = w.q_start + w.L
    if w.mode == "halo":
        # the neighbourhood starts at the first position of the document that
        # holds the shard's first query position (its left straddle)
        d = glob[0, w.q_start]
        s_first = w.q_start
        while s_first > 0 and glob[0, s_first - 1] == d:
            s_first -= 1
        nb_start = s_first
        owner_off = [0, w.q_start - s_first, q_end - s_first]
        owners = [w.cp_rank - 1, w.cp_rank]
    else:
        nb_start = 0
        chunk = w.L
        owner_off = [r * chunk for r in range(w.cp_rank + 2)]
        owners = list(range(w.cp_rank + 1))
    ids = np.ascontiguousarray(glob[:, nb_start:q_end])
    pm = None if pad is None else np.ascontiguousarray(pad[:, nb_start:q_end])
    return DocMap(ids, pm, nb_start, q_end - nb_start, owner_off, owners)


def make_tensors(w: Workload, S: int, dtype: str = "bf16", B: Optional[int] = None):
    """Q [B,Hq,L,D], K/V [B,Hkv,S,D], dO [B,Hq,L,D] as CPU torch tensors.

    ``dtype`` is "bf16" (round-to-nearest-even cast) or "f32" (the debug twin).
    """
    import torch

    B = w.B if B is None else B
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn((B, w.Hq, w.L, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((B, w.Hkv, S, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((B, w.Hkv, S, w.D), generator=g, dtype=torch.float32)
    do = torch.randn((B, w.Hq, w.L, w.D), generator=g, dtype=torch.float32)
    if w.outliers:
        q = torch.where(torch.rand(q.shape, generator=g) < 0.01, q * 8.0, q)
        k = torch.where(torch.rand(k.shape, generator=g) < 0.01, k * 8.0, k)
    if dtype == "bf16":
        q, k, v, do = (t.to(torch.bfloat16) for t in (q, k, v, do))
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v, do


def small_variant(w: Workload, L: int, S_global: int, q_start: int, Hq: Optional[int] = None,
                  Hkv: Optional[int] = None, pad_tail: Optional[int] = None,
                  window: Optional[int] = None, B: Optional[int] = None) -> Workload:
    """Same document law, heads and dtype story at a size the oracle finishes in seconds."""
    kw = dict(w.__dict__)
    kw.update(L=L, S_global=S_global, q_start=q_start)
    if Hq is not None:
        kw["Hq"] = Hq
    if Hkv is not None:
        kw["Hkv"] = Hkv
    if pad_tail is not None:
        kw["pad_tail"] = pad_tail
    if window is not None:
        kw["window"] = window
    if B is not None:
        kw["B"] = B
    if w.mode != "halo":
        kw["cp_rank"] = q_start // L
        kw["cp_size"] = S_global // L
    return Workload(**kw)
