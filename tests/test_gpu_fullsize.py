"""All five workloads at full size, in bf16 and in the float32 debug twin,
through the same C-ABI calls bench.py times, checked against the fp64 oracle on
outputs it can compute exactly one by one:

* segment builder: every array, bit-exact (the integer reference is cheap);
* O, LSE, dQ: sampled query rows (shard edges, document boundaries, random)
  for every q head of the first and last kv head, in every batch row -- each
  row depends only on itself;
* dK, dV, short reductions: sampled keys attended by few query rows, from
  exactly those rows (the sums are complete for them), in every batch row;
* dK, dV, long reductions: the keys with the most attending rows -- the whole
  prefix of the single long document (config 4: every one of its 8192 rows and
  4 heads), the halo keys of the straddling first document (config 3, where
  the key segment is longer than the query segment), the keys reached by a
  whole window (config 2) -- from every attending row.  The oracle runs over
  disjoint row subsets in threads and the partial sums are added (its ``rows``
  argument restricts which rows enter the sums, so the subsets add up to the
  full sum);
* structural zeros: every key no query attends is exactly 0 in dK and dV, and
  padding rows of O / dQ are exactly 0, over the whole tensors;
* owner flags against the oracle's key coverage.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from oracle import nbattn_oracle as orc
from sliding_window_attention_fold_amd import workloads as wl

from gpu_cases import assert_close, check_segments, run_gpu, say, workload_inputs

pytestmark = pytest.mark.gpu


def _sample_rows(inp, seg_ref, b, rng, n_rand=24):
    L = inp.L
    rows = {0, 1, L // 2, L - 2, L - 1}
    n = seg_ref["n_seg"]
    for s in range(n):
        if seg_ref["q_row0"][s] // L != b:
            continue
        r0 = int(seg_ref["q_row0"][s] % L)
        for r in (r0 - 1, r0, r0 + 1):
            if 0 <= r < L:
                rows.add(r)
    rows = sorted(rows)
    if len(rows) > 40:
        rows = sorted(rng.choice(rows, 40, replace=False).tolist())
    rows = sorted(set(rows) | set(rng.integers(0, L, n_rand).tolist()))
    return np.array(rows)


def _bands(inp, seg_ref, b):
    L, S, W = inp.L, inp.S, inp.window
    p = S - L + np.arange(L)
    klo = seg_ref["row_klo"][b * L:(b + 1) * L]
    bs = klo if W < 0 else np.maximum(klo, p - W)
    return bs, p


def _attending(bs, p, j):
    return np.nonzero((bs <= p) & (bs <= j) & (j <= p))[0]


def _sample_keys(inp, seg_ref, b, rng, max_rows=1100):
    """Keys (with the query rows attending them) whose row sets stay small."""
    bs, p = _bands(inp, seg_ref, b)
    S = inp.S
    cand = []
    # the last keys of the neighbourhood, then keys spread over the covered range
    for j in list(range(S - 1, max(S - 40, -1), -7)) + rng.integers(0, S, 400).tolist():
        att = _attending(bs, p, j)
        if 0 < len(att) <= max_rows:
            cand.append((int(j), att))
        if len(cand) >= 12:
            break
    keys = np.array(sorted({j for j, _ in cand}), dtype=np.int64)
    rows = np.unique(np.concatenate([a for _, a in cand])) if cand else np.zeros(0, dtype=np.int64)
    return keys, rows


def _long_keys(inp, seg_ref, b, rng, n_top=8):
    """Keys with the longest reductions: drawn from the keys whose attending-row
    count is at least 90 % of the largest (tile edges first), plus the halo keys
    of a straddling first document and the first keys of the shard."""
    bs, p = _bands(inp, seg_ref, b)
    real = bs <= p
    S, L = inp.S, inp.L
    diff = np.zeros(S + 1, dtype=np.int64)
    np.add.at(diff, bs[real], 1)
    np.add.at(diff, p[real] + 1, -1)
    count = np.cumsum(diff)[:S]
    if count.max() == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
    top = np.nonzero(count >= 0.9 * count.max())[0]
    edges = [j for j in top if j % 64 in (0, 31, 32, 63)]
    pick = set(edges[:: max(1, len(edges) // 4)][:4])
    pick |= set(rng.choice(top, min(n_top, len(top)), replace=False).tolist())
    halo = np.nonzero(count[: S - L] > 0)[0]          # keys before the shard that some row reaches
    if len(halo):
        pick |= {int(halo[0]), int(halo[-1])} | set(rng.choice(halo, min(4, len(halo)), replace=False).tolist())
    pick |= {j for j in (S - L, S - L + 1, S - L + 33) if j < S and count[j] > 0}
    keys = np.array(sorted(pick), dtype=np.int64)
    rows = np.unique(np.concatenate([_attending(bs, p, j) for j in keys]))
    return keys, rows


def _oracle_dkdv(inp, b, kv, g, keys, rows, window, scale):
    """dK, dV of kv head ``kv`` at ``keys`` over the query rows ``rows`` (all of
    the rows attending them), summed over disjoint row subsets run in threads."""
    sl = slice(b, b + 1)
    q = inp.q[sl, kv * g:(kv + 1) * g]
    do = inp.do[sl, kv * g:(kv + 1) * g]
    k = inp.k[sl, kv:kv + 1]
    v = inp.v[sl, kv:kv + 1]
    folded = inp.folded[sl]
    n = max(1, min(8, len(os.sched_getaffinity(0)) // 2, (len(rows) + 255) // 256))
    parts = [r for r in np.array_split(rows, n) if len(r)]

    def one(r):
        _, dK, dV = orc.attention_backward(q, k, v, do, folded, window, scale, kv_heads=[0], rows=r, keys=keys)
        return dK[0, 0, keys], dV[0, 0, keys]

    with threadpool_limits(limits=2), ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(one, parts))
    return sum(x[0] for x in res), sum(x[1] for x in res)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_workload(cfg, dtype):
    w = wl.get(cfg)
    inp = workload_inputs(w, dtype)
    say(f"[full] config {cfg} {dtype}: {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L={w.L} S={inp.S} "
        f"W={w.window}")
    seg, out, lse, res = run_gpu(inp)
    check_segments(seg, inp)
    seg_ref = orc.segments_reference(inp.folded, inp.L, inp.window)
    rng = np.random.default_rng(1000 + cfg + (100 if dtype == "f32" else 0))
    scale = w.D ** -0.5
    real = orc.real_rows(inp.folded, inp.L)

    o_np = out.float().cpu().numpy()
    dq_np = res.dq.float().cpu().numpy()
    dk_np = res.dk.float().cpu().numpy()
    dv_np = res.dv.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    # structural zeros over the whole tensors
    pad_rows = np.broadcast_to(~real[:, None, :], o_np.shape[:3])
    assert (o_np[pad_rows] == 0).all() and (dq_np[pad_rows] == 0).all()
    att = orc.key_attended(inp.folded, inp.L, inp.window)
    unc = np.broadcast_to(~att[:, None, :], dk_np.shape[:3])
    assert (dk_np[unc] == 0).all() and (dv_np[unc] == 0).all()

    for b in range(inp.folded.shape[0]):
        sl = slice(b, b + 1)
        for kv in sorted({0, w.Hkv - 1}):
            heads = list(range(kv * w.g, (kv + 1) * w.g))
            rows = _sample_rows(inp, seg_ref, b, rng)
            O, LSE = orc.attention_forward(inp.q[sl], inp.k[sl], inp.v[sl], inp.folded[sl], w.window, scale,
                                           heads=heads, rows=rows)
            assert_close(f"O b{b} kv{kv}", o_np[sl][:, heads][:, :, rows], O, dtype)
            assert_close(f"LSE b{b} kv{kv}", lse_np[sl][:, heads][:, :, rows], LSE, dtype)
            dQ, _, _ = orc.attention_backward(inp.q[sl], inp.k[sl], inp.v[sl], inp.do[sl], inp.folded[sl],
                                              w.window, scale, kv_heads=[kv], rows=rows,
                                              keys=np.zeros(0, dtype=np.int64))
            assert_close(f"dQ b{b} kv{kv}", dq_np[sl][:, heads][:, :, rows], dQ[:, heads][:, :, rows], dtype)
            keys, krows = _sample_keys(inp, seg_ref, b, rng)
            say(f"[full] config {cfg} {dtype} b {b} kv {kv}: {len(rows)} rows, {len(keys)} short keys from "
                f"{len(krows)} rows")
            if len(keys):
                dK, dV = _oracle_dkdv(inp, b, kv, w.g, keys, krows, w.window, scale)
                assert_close(f"dK short b{b} kv{kv}", dk_np[b, kv, keys], dK, dtype)
                assert_close(f"dV short b{b} kv{kv}", dv_np[b, kv, keys], dV, dtype)
        # long reductions: one kv head per batch row (the last for bf16, the first for f32)
        kv = w.Hkv - 1 if dtype == "bf16" else 0
        keys, krows = _long_keys(inp, seg_ref, b, rng)
        say(f"[full] config {cfg} {dtype} b {b} kv {kv}: {len(keys)} long keys (keys {keys[:3].tolist()}..."
            f"{keys[-3:].tolist()}) from {len(krows)} rows")
        if len(keys):
            dK, dV = _oracle_dkdv(inp, b, kv, w.g, keys, krows, w.window, scale)
            assert_close(f"dK long b{b} kv{kv}", dk_np[b, kv, keys], dK, dtype)
            assert_close(f"dV long b{b} kv{kv}", dv_np[b, kv, keys], dV, dtype)
    # owner flags against the oracle's coverage
    for o, rank in enumerate(inp.owners):
        a, e = inp.owner_off[o], inp.owner_off[o + 1]
        assert res.attended[rank] == bool(att[:, a:e].any())
    torch.cuda.synchronize()
