"""The forward's launch order: the segment builder's fwd_order against a host ranking of the same bands, and
forward results that do not depend on it."""
import numpy as np
import pytest
import torch

import sliding_window_attention_fold_amd as nb
from sliding_window_attention_fold_amd import workloads as wl

from gpu_cases import say

pytestmark = pytest.mark.gpu

ROWS = 128   # rows of one forward query tile


def host_order(row_klo: np.ndarray, B: int, L: int, S: int, W: int) -> np.ndarray:
    """Per batch row, tiles sorted by decreasing work, ties by decreasing index.  A tile's work: the key span of
    each 32-row group's band union plus the span of the tile's union, bands [max(row_klo, p - W), p] at
    p = S - L + i."""
    nq = (L + ROWS - 1) // ROWS
    out = np.empty((B, nq), np.int64)
    for b in range(B):
        if nq > 2048:
            out[b] = np.arange(nq)
            continue
        i = np.arange(L)
        p = S - L + i
        bs = np.maximum(row_klo[b * L:(b + 1) * L].astype(np.int64), 0)
        if W >= 0:
            bs = np.maximum(bs, p - W)
        real = bs <= p
        work = np.zeros(nq, np.int64)
        for t in range(nq):
            ulo, uhi = None, None
            for g in range(0, ROWS, 32):
                r = slice(t * ROWS + g, min(t * ROWS + g + 32, L))
                m = real[r]
                if r.start >= L or not m.any():
                    continue
                lo, hi = bs[r][m].min(), p[r][m].max() + 1
                work[t] += hi - lo
                ulo = lo if ulo is None else min(ulo, lo)
                uhi = hi if uhi is None else max(uhi, hi)
            if ulo is not None:
                work[t] += uhi - ulo
        out[b] = sorted(range(nq), key=lambda t: (-work[t], -t))
    return out


def _docs(rng, S, hi):
    ids, d, x = np.zeros(S, np.int32), 1, 0
    while x < S:
        n = int(rng.integers(1, hi + 1))
        ids[x:x + n] = d
        d += 1
        x += n
    return ids


def test_order_matches_host_ranking():
    rng = np.random.default_rng(7)
    # (the builder ranks up to 256 tiles per batch row by counting and sorts beyond; the last two cases take the
    # sort (313 tiles) and the identity past 2048 tiles)
    cases = [(1, 256, 128, 64), (3, 4000, 1000, -1), (2, 9000, 8193, 700), (1, 300, 1, 0), (4, 8192, 4096, 512),
             (2, 45000, 40000, 900), (1, 270000, 263000, 300)]
    for trial, (B, S, L, W) in enumerate(cases):
        ids = np.stack([_docs(rng, S, int(rng.choice([8, 200, 3000]))) for _ in range(B)])
        pad = (rng.random((B, S)) < 0.05).astype(np.uint8) if trial % 2 else None
        say(f"[fwd order] case {trial} B={B} S={S} L={L} W={W}")
        seg = nb.segment_build(torch.from_numpy(ids).cuda(), L, W,
                               None if pad is None else torch.from_numpy(pad).cuda())
        got = seg.fwd_order.cpu().numpy().reshape(B, -1)
        want = host_order(seg.row_klo.cpu().numpy(), B, L, S, W)
        assert np.array_equal(got, want)


def test_order_leaves_results_unchanged():
    """Config 5's map (1024 forward workgroups: more than one round) launched in the builder's order and in grid
    order (the identity written over fwd_order) gives bitwise the same O and LSE."""
    w = wl.get(5)
    dm = wl.make_doc_map(w)
    q, k, v, _ = wl.make_tensors(w, dm.S, "bf16")
    dev = torch.device("cuda:0")
    say("[fwd order] config 5 map, ordered vs grid order")
    seg = nb.segment_build(torch.from_numpy(dm.doc_ids).to(dev), w.L, w.window,
                           None if dm.pad_mask is None else torch.from_numpy(dm.pad_mask).to(dev))
    order = seg.fwd_order.cpu().numpy().reshape(w.B, -1)
    assert not np.array_equal(order, np.broadcast_to(np.arange(order.shape[1]), order.shape))
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    o1, s1 = nb.attn_fwd(qd, kd, vd, seg)
    seg.fwd_order.copy_(torch.arange(order.shape[1], dtype=torch.int32, device=dev).repeat(w.B))
    o2, s2 = nb.attn_fwd(qd, kd, vd, seg)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1.lse, s2.lse)


@pytest.mark.parametrize("B, W, per_cu", [(1, 600, 2), (2, 300, 3)])
def test_multi_round_forward_full_parity(B, W, per_cu):
    """A forward whose grid exceeds one round of workgroups runs in the builder's order; O, LSE and the gradients
    match the oracle element by element.  At D = 128 the forward takes two workgroups per CU with 64-key tiles,
    and three per CU with 32-key tiles when the left window is at most 512 keys: 18 query tiles x 32 heads x B
    workgroups against per_cu workgroups per CU."""
    from gpu_cases import custom_inputs, full_parity

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    Hq, Hkv, D, L, S = 32, 8, 128, 2200, 2600
    assert ((L + ROWS - 1) // ROWS) * Hq * B > per_cu * n_cu, "the grid must take more than one round here"
    rng = np.random.default_rng(11)
    ids = np.stack([_docs(rng, S, 400) for _ in range(B)])
    # padding as whole documents (every 7th) and a tail: every document stays one run of its id
    ids[np.isin(ids, np.arange(7, ids.max() + 1, 7))] = 0
    pad = np.zeros((B, S), np.uint8)
    pad[:, -60:] = 1
    say(f"[fwd order] multi-round forward B={B} Hq={Hq} Hkv={Hkv} D={D} L={L} S={S} W={W}")
    seg = nb.segment_build(torch.from_numpy(ids).cuda(), L, W, torch.from_numpy(pad).cuda())
    assert seg.header_host()["status"] == 0
    order = seg.fwd_order.cpu().numpy().reshape(B, -1)
    assert not np.array_equal(order, np.broadcast_to(np.arange(order.shape[1]), order.shape)), \
        "the order should differ from grid order"
    full_parity(custom_inputs(ids, pad, Hq, Hkv, D, L, W, "bf16", seed=5), "bf16")
