"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each check is independent of the oracle's own code path: hand-worked values,
closed forms, a library routine on the special case it reduces to, a
pure-Python scalar loop, finite differences, torch autograd, and the
full-sequence / simulated-ring identities the pages state.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import nbattn_oracle as orc
from sliding_window_attention_fold_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_by_hand.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _rand_docmap(rng, B, S, pad_tail=0, lo=1, hi=6):
    ids = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        pos, d = 0, 1
        while pos < S:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    if pad_tail:
        ids[:, S - pad_tail:] = 0
    return ids


# ----------------------------------------------------------------------------- fold / mask

def test_fold_pad():
    ids = np.array([[3, 3, 4, 4, 5]])
    pm = np.array([[0, 0, 0, 1, 1]], dtype=np.uint8)
    assert orc.fold_pad(ids, pm).tolist() == [[3, 3, 4, 0, 0]]
    assert orc.fold_pad(ids, None).tolist() == ids.tolist()


def _interval_mask(folded, L, W):
    """Independent form: a real row at p allows exactly [max(run_start(p), p-W), p]; pad rows only p."""
    B, S = folded.shape
    M = np.zeros((B, 1, L, S), dtype=bool)
    for b in range(B):
        for i in range(L):
            p = S - L + i
            d = folded[b, p]
            if d <= 0:
                M[b, 0, i, p] = True
                continue
            a = p
            while a > 0 and folded[b, a - 1] == d:
                a -= 1
            lo = a if W < 0 else max(a, p - W)
            M[b, 0, i, lo:p + 1] = True
    return M


@pytest.mark.parametrize("seed", range(6))
def test_mask_equals_interval_form(seed):
    rng = np.random.default_rng(seed)
    S, L = 40, 24
    ids = _rand_docmap(rng, 2, S, pad_tail=int(rng.integers(0, 5)))
    W = int(rng.choice([-1, 0, 1, 3, 7, 100]))
    assert np.array_equal(orc.allow_mask(ids, L, W), _interval_mask(ids, L, W))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_mask_invariants_on_workloads(cfg):
    """Mask invariants on each workload's real doc map, checked per row block
    (every row block, except config 4 -- one 65536-key document -- where the first,
    middle and last blocks are checked)."""
    w = wl.get(cfg)
    dm = wl.make_doc_map(w)
    f = orc.fold_pad(dm.doc_ids, dm.pad_mask)
    B, S = f.shape
    L = w.L
    j = np.arange(S)
    step = 512
    starts = list(range(0, L, step))
    if L * S > (1 << 26):
        starts = sorted({starts[0], starts[len(starts) // 2], starts[-1]})
    for b in range(B):
        for s0 in starts:
            rows = np.arange(s0, min(L, s0 + step))
            M = orc.allow_mask(f[b:b + 1], L, w.window, rows=rows)[0, 0]
            p = S - L + rows
            r = np.arange(len(rows))
            # diagonal always allowed
            assert M[r, p].all()
            off = M.copy()
            off[r, p] = False
            fp = f[b, p][:, None]
            ok = (j[None, :] <= p[:, None]) & (f[b][None, :] == fp) & (fp > 0)   # causal, same doc, not padding
            if w.window >= 0:
                ok &= (p[:, None] - j[None, :]) <= w.window                      # inside the window
            assert not (off & ~ok).any()
            # pad rows: only the (harmless) diagonal
            assert not off[f[b, p] <= 0].any()


def test_mask_is_full_sequence_slice():
    """_cp_blockdiag_mask: local rows equal the non-CP packed mask's rows at their global positions."""
    rng = np.random.default_rng(7)
    ids = _rand_docmap(rng, 1, 48, pad_tail=5)
    for W in (-1, 4):
        full = orc.allow_mask(ids, 48, W)[0, 0]
        for L in (1, 13, 30, 48):
            assert np.array_equal(orc.allow_mask(ids, L, W)[0, 0], full[48 - L:])


# ----------------------------------------------------------------------------- segments

@pytest.mark.parametrize("case", range(4))
def test_segments_hand_worked(case):
    g = _gold()["segments"][case]
    f = np.array(g["folded"])
    seg = orc.segments_reference(f, g["L"], g["window"])
    for key in ("n_seg", "lo", "max_q", "max_k", "status"):
        assert seg[key] == g[key], key
    for key in ("cu_q", "cu_k", "q_row0", "k_row0", "row_seg", "row_klo", "kcov_lo"):
        assert seg[key].tolist() == g[key], key
    assert orc.useful_pairs(f, g["L"], g["window"]) == g["pairs"]


@pytest.mark.parametrize("seed", range(8))
def test_segment_invariants_and_coverage(seed):
    rng = np.random.default_rng(100 + seed)
    B, S = 2, int(rng.integers(8, 60))
    L = int(rng.integers(1, S + 1))
    W = int(rng.choice([-1, 0, 2, 5, 1000]))
    f = _rand_docmap(rng, B, S, pad_tail=int(rng.integers(0, 4)), lo=1, hi=int(rng.integers(1, 12)))
    seg = orc.segments_reference(f, L, W)
    n = seg["n_seg"]
    ql = np.diff(seg["cu_q"])
    kl = np.diff(seg["cu_k"])
    real = orc.real_rows(f, L).reshape(-1)
    # q segments partition the real rows
    covered = np.zeros(B * L, dtype=int)
    for s in range(n):
        covered[seg["q_row0"][s]:seg["q_row0"][s] + ql[s]] += 1
    assert np.array_equal(covered, real.astype(int))
    assert np.array_equal(seg["row_seg"] >= 0, real)
    for s in range(n):
        b = seg["q_row0"][s] // L
        q0 = seg["q_row0"][s] - b * L
        k0 = seg["k_row0"][s] - b * S
        # key end equals query end (bottom-right alignment), sk >= sq
        assert k0 + kl[s] == S - L + q0 + ql[s]
        assert kl[s] >= ql[s] >= 1
        # key start is the run start clipped at lo
        a = S - L + q0
        while a > 0 and f[b, a - 1] == f[b, S - L + q0]:
            a -= 1
        assert k0 == max(a, seg["lo"])
    assert seg["max_q"] == (ql.max() if n else 0) and seg["max_k"] == (kl.max() if n else 0)
    # the covered key set equals the set of keys the mask lets some real row attend
    att = orc.key_attended(f, L, W)
    cov = np.zeros((B, S), dtype=bool)
    for s in range(n):
        b = seg["k_row0"][s] // S
        k0 = seg["k_row0"][s] - b * S
        cov[b, k0:k0 + kl[s]] = True
    assert np.array_equal(att, cov)
    # kcov_lo is the first covered key
    for b in range(B):
        nz = np.nonzero(cov[b])[0]
        assert seg["kcov_lo"][b] == (nz[0] if len(nz) else S)
    # useful pairs: sum over real rows of the band length [max(row_klo, p-W), p]
    p = S - L + np.tile(np.arange(L), B)
    lo = seg["row_klo"] if W < 0 else np.maximum(seg["row_klo"], p - W)
    assert orc.useful_pairs(f, L, W) == int(np.where(real, p - lo + 1, 0).sum())


def test_pairs_closed_form_single_document():
    """One document over 65536 positions, L = 8192 suffix, no window: sum_{i<8192} (57345 + i)."""
    w = wl.get(4)
    f = orc.fold_pad(wl.make_doc_map(w).doc_ids, None)
    expect = sum(57345 + i for i in range(8192))
    assert expect == 503_320_576
    assert orc.useful_pairs(f, w.L, w.window, row_block=1024) == expect


# ----------------------------------------------------------------------------- forward

@pytest.mark.parametrize("case", range(4))
def test_forward_hand_worked(case):
    g = _gold()["attention"][case]
    O, LSE = orc.attention_forward(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                                   np.array(g["folded"]), g["window"], g["scale"])
    assert np.allclose(O, np.array(g["O"]), atol=1e-12)
    assert np.allclose(np.exp(LSE), np.array(g["LSE_exp"]), atol=1e-12)


def _rand_qkv(rng, B, Hq, Hkv, L, S, D, scale_q=1.0):
    q = rng.standard_normal((B, Hq, L, D)) * scale_q
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    return q, k, v


def test_forward_matches_torch_sdpa_single_doc():
    """One document, no padding, no window, S = L: plain causal SDPA with GQA (fp64, CPU)."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, L, D = 2, 4, 2, 37, 16
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, L, D)
    f = np.ones((B, L), dtype=np.int64)
    scale = D ** -0.5
    O, LSE = orc.attention_forward(q, k, v, f, -1, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        scale=scale, enable_gqa=True)
    assert np.allclose(O, ref.numpy(), atol=1e-12)
    # LSE: logsumexp of the causal scores, by torch
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    s = scale * torch.from_numpy(q) @ kk.transpose(-1, -2)
    s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    assert np.allclose(LSE, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def _scalar_loop_forward(q, k, v, f, W, scale):
    """Pure-Python per-element attention straight from the mask definition."""
    B, Hq, L, D = q.shape
    S = k.shape[2]
    g = Hq // k.shape[1]
    O = np.zeros_like(q)
    LSE = np.full((B, Hq, L), -math.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(L):
                p = S - L + i
                if f[b, p] <= 0:
                    continue
                keys = [j for j in range(S) if f[b, j] == f[b, p] and j <= p and (W < 0 or p - j <= W)]
                sc = [scale * sum(q[b, h, i, d] * k[b, h // g, j, d] for d in range(D)) for j in keys]
                m = max(sc)
                z = sum(math.exp(x - m) for x in sc)
                LSE[b, h, i] = m + math.log(z)
                for jj, j in enumerate(keys):
                    w = math.exp(sc[jj] - LSE[b, h, i])
                    for d in range(D):
                        O[b, h, i, d] += w * v[b, h // g, j, d]
    return O, LSE


@pytest.mark.parametrize("seed", range(3))
def test_forward_matches_scalar_loop(seed):
    rng = np.random.default_rng(20 + seed)
    B, Hq, Hkv, S, L, D = 2, 4, 2, 19, 11, 3
    f = _rand_docmap(rng, B, S, pad_tail=2, lo=1, hi=7)
    W = [-1, 2, 5][seed]
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    O, LSE = orc.attention_forward(q, k, v, f, W, 0.7)
    O2, LSE2 = _scalar_loop_forward(q, k, v, f, W, 0.7)
    assert np.allclose(O, O2, atol=1e-12)
    assert np.array_equal(np.isinf(LSE), np.isinf(LSE2))
    fin = np.isfinite(LSE2)
    assert np.allclose(LSE[fin], LSE2[fin], atol=1e-12)


def test_forward_closed_forms():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, S, L, D = 1, 4, 2, 30, 20, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    f = _rand_docmap(rng, B, S, pad_tail=3, lo=2, hi=9)
    real = orc.real_rows(f, L)[0]
    g = Hq // Hkv
    # window 0: O_i = v_p, LSE_i = scale q_i . k_p (real rows); pad rows 0 / -inf
    O, LSE = orc.attention_forward(q, k, v, f, 0, 0.3)
    for h in range(Hq):
        exp_o = v[0, h // g, S - L:]
        exp_l = 0.3 * np.einsum("id,id->i", q[0, h], k[0, h // g, S - L:])
        assert np.allclose(O[0, h][real], exp_o[real], atol=1e-12)
        assert np.allclose(LSE[0, h][real], exp_l[real], atol=1e-12)
        assert (O[0, h][~real] == 0).all() and np.isneginf(LSE[0, h][~real]).all()
    # documents of length 1 give the same closed form without a window
    f1 = np.arange(1, S + 1)[None, :]
    O1, LSE1 = orc.attention_forward(q, k, v, f1, -1, 0.3)
    O0, LSE0 = orc.attention_forward(q, k, v, f1, 0, 0.3)
    assert np.allclose(O1, O0) and np.allclose(LSE1, LSE0)
    # window >= S equals no window
    Oa, La = orc.attention_forward(q, k, v, f, S, 0.3)
    Ob, Lb = orc.attention_forward(q, k, v, f, -1, 0.3)
    assert np.array_equal(Oa, Ob) and np.array_equal(La, Lb)


def test_forward_is_full_sequence_slice():
    """Local rows equal rows [S-L, S) of the full-sequence attention (non-CP run)."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, S, D = 2, 2, 1, 33, 5
    f = _rand_docmap(rng, B, S, pad_tail=4, lo=2, hi=10)
    q_full, k, v = _rand_qkv(rng, B, Hq, Hkv, S, S, D)
    for W in (-1, 6):
        Of, Lf = orc.attention_forward(q_full, k, v, f, W, 0.5)
        for L in (1, 9, 20):
            O, LSE = orc.attention_forward(q_full[:, :, S - L:], k, v, f, W, 0.5)
            assert np.allclose(O, Of[:, :, S - L:], atol=1e-13)
            assert np.array_equal(np.isinf(LSE), np.isinf(Lf[:, :, S - L:]))
            fin = np.isfinite(LSE)
            assert np.allclose(LSE[fin], Lf[:, :, S - L:][fin], atol=1e-13)


def test_forward_large_scores_stay_finite():
    """Max subtraction: scores far beyond exp's range still give finite O/LSE."""
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 6, 10, 4)
    f = np.ones((1, 10), dtype=np.int64)
    O, LSE = orc.attention_forward(q * 400, k, v, f, -1, 1.0)
    assert np.isfinite(O).all() and np.isfinite(LSE).all()


def test_forward_subset_rows_heads():
    rng = np.random.default_rng(6)
    q, k, v = _rand_qkv(rng, 2, 4, 2, 12, 20, 4)
    f = _rand_docmap(rng, 2, 20, pad_tail=2)
    O, LSE = orc.attention_forward(q, k, v, f, 3, 0.5)
    rows, heads = [0, 5, 11], [1, 3]
    Os, Ls = orc.attention_forward(q, k, v, f, 3, 0.5, heads=heads, rows=rows, row_block=2)
    assert np.array_equal(Os, O[:, heads][:, :, rows])
    assert np.array_equal(Ls, LSE[:, heads][:, :, rows])


# ----------------------------------------------------------------------------- backward

def _loss(q, k, v, dout, f, W, scale):
    O, _ = orc.attention_forward(q, k, v, f, W, scale)
    return float((O * dout).sum())


def test_backward_finite_differences():
    """Central differences, fp64, h = 1e-6, on B=1, Hq=2, Hkv=1, D=4, S=10, L=6, 3 docs, one pad row, W=3."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, S, L, D = 1, 2, 1, 10, 6, 4
    f = np.array([[1, 1, 1, 2, 2, 2, 2, 3, 3, 0]])
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    dout = rng.standard_normal((B, Hq, L, D))
    W, scale, h = 3, 0.5, 1e-6
    dQ, dK, dV = orc.attention_backward(q, k, v, dout, f, W, scale)
    for name, x, gx in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, dout, f, W, scale)
            x[idx] = old - h
            lm = _loss(q, k, v, dout, f, W, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - gx).max() / max(1e-30, np.abs(gx).max())
        assert err <= 1e-6, (name, err)
    # padding row: dQ = 0
    assert (dQ[0, :, 5] == 0).all()


def _torch_dense(q, k, v, f, W, scale):
    """Dense masked softmax attention in torch fp64 (autograd), built from the mask definition."""
    B, Hq, L, D = q.shape
    g = Hq // k.shape[1]
    M = torch.from_numpy(orc.allow_mask(f, L, W))
    real = torch.from_numpy(orc.real_rows(f, L))[:, None, :, None]
    kk = k.repeat_interleave(g, dim=1)
    vv = v.repeat_interleave(g, dim=1)
    s = scale * q @ kk.transpose(-1, -2)
    s = s.masked_fill(~M, float("-inf"))
    o = torch.softmax(s, -1) @ vv
    return torch.where(real, o, torch.zeros_like(o))


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_torch_autograd(seed):
    rng = np.random.default_rng(30 + seed)
    B, Hq, Hkv, S, L, D = 2, 4, 2, 26, 17, 6
    f = _rand_docmap(rng, B, S, pad_tail=3, lo=1, hi=8)
    W = [-1, 4, 0][seed]
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    dout = rng.standard_normal((B, Hq, L, D))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = _torch_dense(tq, tk, tv, f, W, 0.4)
    (o * torch.from_numpy(dout)).sum().backward()
    dQ, dK, dV = orc.attention_backward(q, k, v, dout, f, W, 0.4)
    assert np.allclose(dQ, tq.grad.numpy(), atol=1e-12)
    assert np.allclose(dK, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dV, tv.grad.numpy(), atol=1e-12)


def test_backward_matches_sdpa_autograd_single_doc():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, L, D = 1, 4, 1, 21, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, L, D)
    dout = rng.standard_normal((B, Hq, L, D))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.35,
                                                         enable_gqa=True)
    (o * torch.from_numpy(dout)).sum().backward()
    dQ, dK, dV = orc.attention_backward(q, k, v, dout, np.ones((1, L), dtype=np.int64), -1, 0.35)
    assert np.allclose(dQ, tq.grad.numpy(), atol=1e-12)
    assert np.allclose(dK, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dV, tv.grad.numpy(), atol=1e-12)


def test_backward_window_zero_closed_form():
    """W = 0: O_i = v_p, so dQ = 0, dK = 0 and dV_p = sum over the group's heads of dO."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, S, L, D = 1, 4, 2, 14, 9, 5
    f = _rand_docmap(rng, B, S, pad_tail=2)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    dout = rng.standard_normal((B, Hq, L, D))
    dQ, dK, dV = orc.attention_backward(q, k, v, dout, f, 0, 0.5)
    real = orc.real_rows(f, L)[0]
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    for kv in range(Hkv):
        expect = np.zeros((S, D))
        expect[S - L:][real] = dout[0, 2 * kv:2 * kv + 2].sum(0)[real]
        assert np.allclose(dV[0, kv], expect, atol=1e-14)


@pytest.mark.parametrize("W", [-1, 5])
def test_simulated_ring_owner_sums(W):
    """_route_kv_grads_to_owners: each owner's dK/dV summed over the ranks that attended it equals
    the full-sequence gradient; each rank's output equals its rows of the full-sequence output."""
    rng = np.random.default_rng(11)
    cp, Lc, B, Hq, Hkv, D = 4, 8, 1, 2, 1, 3
    S = cp * Lc
    f = _rand_docmap(rng, B, S, pad_tail=3, lo=2, hi=11)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, S, S, D)
    dout = rng.standard_normal((B, Hq, S, D))
    O_full, _ = orc.attention_forward(q, k, v, f, W, 0.6)
    dQ_full, dK_full, dV_full = orc.attention_backward(q, k, v, dout, f, W, 0.6)
    dK_sum = np.zeros_like(k)
    dV_sum = np.zeros_like(v)
    for r in range(cp):
        Snb = (r + 1) * Lc
        fr = f[:, :Snb]
        sl = slice(r * Lc, (r + 1) * Lc)
        O, _ = orc.attention_forward(q[:, :, sl], k[:, :, :Snb], v[:, :, :Snb], fr, W, 0.6)
        assert np.allclose(O, O_full[:, :, sl], atol=1e-13)
        dQ, dK, dV = orc.attention_backward(q[:, :, sl], k[:, :, :Snb], v[:, :, :Snb],
                                            dout[:, :, sl], fr, W, 0.6)
        assert np.allclose(dQ, dQ_full[:, :, sl], atol=1e-13)
        att = orc.key_attended(fr, Lc, W)
        off = [o * Lc for o in range(r + 2)]
        dk_l, dv_l, attended = orc.owner_split(dK, dV, off, att)
        for o in range(r + 1):
            if not attended[o]:
                assert (dk_l[o] == 0).all() and (dv_l[o] == 0).all()
            dK_sum[:, :, o * Lc:(o + 1) * Lc] += dk_l[o]
            dV_sum[:, :, o * Lc:(o + 1) * Lc] += dv_l[o]
    assert np.allclose(dK_sum, dK_full, atol=1e-12)
    assert np.allclose(dV_sum, dV_full, atol=1e-12)


def test_owner_split_zeros_and_sum():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, L, D = 1, 2, 1, 40, 10, 3
    f = _rand_docmap(rng, B, S, lo=3, hi=5)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    dout = rng.standard_normal((B, Hq, L, D))
    _, dK, dV = orc.attention_backward(q, k, v, dout, f, 2, 0.5)
    att = orc.key_attended(f, L, 2)
    off = [0, 10, 20, 30, 40]
    dk_l, dv_l, attended = orc.owner_split(dK, dV, off, att)
    indep = _interval_mask(f, L, 2)[0, 0][orc.real_rows(f, L)[0]].any(axis=0)
    assert attended == [bool(indep[a:a + 10].any()) for a in off[:-1]]
    assert attended[:2] == [False, False] and attended[3]
    assert all((x == 0).all() for x in dk_l[:2] + dv_l[:2])
    assert np.array_equal(np.concatenate(dk_l, axis=2), dK)
    # keys outside the attended set are exact zeros
    assert (dK[:, :, ~att[0]] == 0).all() and (dV[:, :, ~att[0]] == 0).all()


def test_backward_row_and_key_restriction():
    """Restricting the sums to the rows that attend a key set gives the full result at those keys."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, S, L, D = 1, 2, 1, 30, 20, 4
    f = _rand_docmap(rng, B, S, pad_tail=2, lo=2, hi=8)
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, S, D)
    dout = rng.standard_normal((B, Hq, L, D))
    dQ, dK, dV = orc.attention_backward(q, k, v, dout, f, 3, 0.5)
    keys = np.array([12, 20, 27])
    M = orc.allow_mask(f, L, 3)[0, 0] & orc.real_rows(f, L)[0][:, None]
    rows = np.nonzero(M[:, keys].any(axis=1))[0]
    dQ2, dK2, dV2 = orc.attention_backward(q, k, v, dout, f, 3, 0.5, rows=rows, keys=keys, row_block=2)
    assert np.allclose(dK2[:, :, keys], dK[:, :, keys], atol=1e-14)
    assert np.allclose(dV2[:, :, keys], dV[:, :, keys], atol=1e-14)
    assert np.allclose(dQ2[:, :, rows], dQ[:, :, rows], atol=1e-14)
    other = np.setdiff1d(np.arange(S), keys)
    assert (dK2[:, :, other] == 0).all()
