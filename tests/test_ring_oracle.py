"""Pins of the ring-attention oracle (CPU only).

Each check holds independently of the ring oracle's own code: the merged ring
result must equal one softmax over the whole causal neighbourhood (the pinned
neighbourhood-attention oracle over the concatenated chunks, no window); the
chunks' backward contributions must add up to that attention's analytic
gradients and split its dK/dV by owner; the merge must reproduce the closed
form of a two-key softmax, treat a row neither side covers as 0 without NaN,
and be commutative and associative; the live-row merge must equal the dense
merge on its rows and leave every other row alone.
"""
import numpy as np
import pytest

from oracle import nbattn_oracle as orc
from oracle import ring_oracle as ro


def _ids(rng, B, N, lo, hi, pad_tail=0):
    ids = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        pos, d = 0, 1
        while pos < N:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
        if pad_tail:
            ids[b, N - pad_tail:] = 0
    return ids


def _world(seed, B, Hq, Hkv, D, Lc, P, lo, hi, pad_tail=0):
    rng = np.random.default_rng(seed)
    ids = _ids(rng, B, P * Lc, lo, hi, pad_tail)
    q_all = rng.standard_normal((B, Hq, P * Lc, D))
    k_all = rng.standard_normal((B, Hkv, P * Lc, D))
    v_all = rng.standard_normal((B, Hkv, P * Lc, D))
    do_all = rng.standard_normal((B, Hq, P * Lc, D))
    return ids, q_all, k_all, v_all, do_all


CASES = [  # seed, B, Hq, Hkv, D, Lc, P, rank, doc lengths lo..hi, pad tail
    (1, 1, 2, 1, 8, 12, 3, 2, 2, 9, 0),
    (2, 2, 4, 2, 16, 10, 4, 3, 1, 30, 5),
    (3, 1, 2, 2, 8, 16, 2, 1, 40, 60, 0),     # one document over both chunks
    (4, 2, 2, 1, 4, 7, 5, 4, 1, 3, 3),        # many short documents
    (5, 1, 4, 1, 8, 9, 3, 0, 3, 12, 0),       # rank 0: the local chunk only
]


@pytest.mark.parametrize("case", CASES)
def test_ring_forward_is_one_softmax_over_the_neighbourhood(case):
    seed, B, Hq, Hkv, D, Lc, P, r, lo, hi, pt = case
    ids, q_all, k_all, v_all, _ = _world(seed, B, Hq, Hkv, D, Lc, P, lo, hi, pt)
    scale = D ** -0.5
    q = q_all[:, :, r * Lc:(r + 1) * Lc]
    kc = [k_all[:, :, o * Lc:(o + 1) * Lc] for o in range(r + 1)]
    vc = [v_all[:, :, o * Lc:(o + 1) * Lc] for o in range(r + 1)]
    out, lse = ro.ring_forward(q, kc, vc, ids, r, scale)
    S = (r + 1) * Lc
    o_ref, l_ref = orc.attention_forward(q, k_all[:, :, :S], v_all[:, :, :S], ids[:, :S], -1, scale)
    assert np.allclose(out, o_ref, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.allclose(lse[fin], l_ref[fin], rtol=1e-12, atol=1e-12)
    assert np.all(out[~fin] == 0)


@pytest.mark.parametrize("case", CASES)
def test_ring_backward_adds_up_to_the_neighbourhood_gradients(case):
    seed, B, Hq, Hkv, D, Lc, P, r, lo, hi, pt = case
    ids, q_all, k_all, v_all, do_all = _world(seed, B, Hq, Hkv, D, Lc, P, lo, hi, pt)
    scale = D ** -0.5
    q = q_all[:, :, r * Lc:(r + 1) * Lc]
    do = do_all[:, :, r * Lc:(r + 1) * Lc]
    kc = [k_all[:, :, o * Lc:(o + 1) * Lc] for o in range(r + 1)]
    vc = [v_all[:, :, o * Lc:(o + 1) * Lc] for o in range(r + 1)]
    out, lse = ro.ring_forward(q, kc, vc, ids, r, scale)
    dq, dks, dvs = ro.ring_backward(q, kc, vc, do, out, lse, ids, r, scale)
    S = (r + 1) * Lc
    dq_ref, dk_ref, dv_ref = orc.attention_backward(q, k_all[:, :, :S], v_all[:, :, :S], do, ids[:, :S], -1, scale)
    assert np.allclose(dq, dq_ref, rtol=1e-10, atol=1e-10)
    for o in range(r + 1):
        assert np.allclose(dks[o], dk_ref[:, :, o * Lc:(o + 1) * Lc], rtol=1e-10, atol=1e-10)
        assert np.allclose(dvs[o], dv_ref[:, :, o * Lc:(o + 1) * Lc], rtol=1e-10, atol=1e-10)


def test_chunk_masks_are_the_neighbourhood_mask_restricted_to_the_chunk():
    rng = np.random.default_rng(9)
    Lc, P = 11, 4
    ids = _ids(rng, 2, P * Lc, 1, 25, 4)
    r = 3
    q_ids = ids[:, r * Lc:]
    # [B, Lc, (r+1) Lc]; padding query rows (whose diagonal the block-diagonal
    # mask keeps, the rows being dropped afterwards) have no keys in a chunk
    full = orc.allow_mask(ids[:, :(r + 1) * Lc], Lc, -1)[:, 0] & (q_ids > 0)[:, :, None]
    for o in range(r + 1):
        M = ro.chunk_mask(q_ids, ids[:, o * Lc:(o + 1) * Lc], r * Lc, o * Lc, o == r)
        assert np.array_equal(M, full[:, :, o * Lc:(o + 1) * Lc])
    # a cross chunk is non-causal: every key precedes every query, so the
    # causal cut changes nothing there
    M0 = ro.chunk_mask(q_ids, ids[:, :Lc], r * Lc, 0, True)
    assert np.array_equal(M0, ro.chunk_mask(q_ids, ids[:, :Lc], r * Lc, 0, False))


def test_merge_two_key_closed_form():
    # one row, keys with scores s1, s2 and values v1, v2 in separate chunks
    s1, s2 = 0.3, -1.7
    v1, v2 = np.array([1.0, -2.0, 0.5]), np.array([4.0, 0.25, -1.0])
    o1, l1 = v1[None, None, None], np.array([[[s1]]])
    o2, l2 = v2[None, None, None], np.array([[[s2]]])
    out, lse = ro.merge(o1, l1, o2, l2)
    w1, w2 = np.exp(s1), np.exp(s2)
    assert np.allclose(out[0, 0, 0], (w1 * v1 + w2 * v2) / (w1 + w2), rtol=1e-15, atol=1e-15)
    assert np.isclose(lse[0, 0, 0], np.log(w1 + w2), rtol=1e-15, atol=1e-15)


def test_merge_edge_rows_and_identities():
    rng = np.random.default_rng(4)
    shape = (2, 3, 5)
    oa, ob, oc = (rng.standard_normal(shape + (4,)) for _ in range(3))
    la, lb, lc = (rng.standard_normal(shape) * 3 for _ in range(3))
    la[0, 0, 0] = lb[0, 0, 0] = -np.inf        # covered by neither side
    oa[0, 0, 0] = ob[0, 0, 0] = 0.0
    lb[1, 2, 3] = -np.inf                       # covered by one side only
    ob[1, 2, 3] = 0.0
    out, lse = ro.merge(oa, la, ob, lb)
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    assert np.all(out[0, 0, 0] == 0) and lse[0, 0, 0] == -np.inf
    assert np.allclose(out[1, 2, 3], oa[1, 2, 3]) and np.isclose(lse[1, 2, 3], la[1, 2, 3])
    # nothing merged yet / an empty accumulator
    o0, l0 = ro.merge(None, None, ob, lb)
    assert np.array_equal(o0, ob) and np.array_equal(l0, lb)
    o1, l1 = ro.merge(np.zeros_like(ob), np.full(shape, -np.inf), ob, lb)
    assert np.allclose(o1, ob, rtol=1e-15, atol=1e-15) and np.array_equal(l1, lb)
    # commutative and associative
    ox, lx = ro.merge(ob, lb, oa, la)
    assert np.allclose(ox, out, rtol=1e-14, atol=1e-14) and np.allclose(lx, lse, rtol=1e-14, atol=1e-14)
    o_ab_c = ro.merge(*ro.merge(oa, la, ob, lb), oc, lc)
    o_a_bc = ro.merge(oa, la, *ro.merge(ob, lb, oc, lc))
    assert np.allclose(o_ab_c[0], o_a_bc[0], rtol=1e-13, atol=1e-13)
    assert np.allclose(o_ab_c[1], o_a_bc[1], rtol=1e-13, atol=1e-13)


def test_merge_live_equals_dense_merge_on_its_rows():
    rng = np.random.default_rng(5)
    B, H, S, D = 2, 3, 9, 4
    oa, ob = rng.standard_normal((B, H, S, D)), rng.standard_normal((B, H, S, D))
    la, lb = rng.standard_normal((B, H, S)), rng.standard_normal((B, H, S))
    idx = np.array([0, 4, 8, 9, 13, 17])
    o, l = ro.merge_live(oa, la, ob, lb, idx)
    od, ld = ro.merge(oa, la, ob, lb)
    mask = np.zeros(B * S, dtype=bool)
    mask[idx] = True
    mask = mask.reshape(B, S)
    for b in range(B):
        for s in range(S):
            if mask[b, s]:
                assert np.allclose(o[b, :, s], od[b, :, s], rtol=1e-15, atol=1e-15)
                assert np.allclose(l[b, :, s], ld[b, :, s], rtol=1e-15, atol=1e-15)
            else:
                assert np.array_equal(o[b, :, s], oa[b, :, s]) and np.array_equal(l[b, :, s], la[b, :, s])


def test_a_planted_merge_mistake_is_caught():
    """The neighbourhood check fails for a merge that forgets to renormalise the
    accumulator (weight 1 instead of exp(lse_acc - lse))."""
    ids, q_all, k_all, v_all, _ = _world(3, 1, 2, 2, 8, 16, 2, 40, 60, 0)
    scale = 8 ** -0.5
    q = q_all[:, :, 16:]
    kc = [k_all[:, :, :16], k_all[:, :, 16:]]
    vc = [v_all[:, :, :16], v_all[:, :, 16:]]
    so, sl = ro.chunk_forward(q, kc[1], vc[1], ids[:, 16:], ids[:, 16:], 16, 16, True, scale)
    co, cl = ro.chunk_forward(q, kc[0], vc[0], ids[:, 16:], ids[:, :16], 16, 0, False, scale)
    lse = np.logaddexp(sl, cl)
    wrong = so + np.exp(cl - lse)[..., None] * co
    o_ref, _ = orc.attention_forward(q, k_all, v_all, ids, -1, scale)
    assert not np.allclose(wrong, o_ref, rtol=1e-6, atol=1e-6)
    right, _ = ro.merge(so, sl, co, cl)
    assert np.allclose(right, o_ref, rtol=1e-12, atol=1e-12)
