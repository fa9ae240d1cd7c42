"""Pins of the exchange-plan oracle (CPU only).

Each check holds independently of the oracle's own code: closed forms for
special document layouts, the attention mask the exchange must serve (the
range is exactly the keys a rank's real queries attend), the workload
generator's own straddle computation, the gather's closed form and the
backward's adjointness.
"""
import numpy as np
import pytest

from oracle import exchange_oracle as ex
from sliding_window_attention_fold_amd import workloads as wl


def _rand_ids(rng, B, N, lo, hi, pad_tail=0, same_rows=False):
    ids = np.zeros((B, N), dtype=np.int64)
    for b in range(B):
        if same_rows and b:
            ids[b] = ids[0]
            continue
        pos, d = 0, 1
        while pos < N:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    pad = None
    if pad_tail:
        pad = np.zeros((B, N), dtype=np.uint8)
        pad[:, N - pad_tail:] = 1
    return ids, pad


def test_single_document_closed_form():
    cp, L = 4, 8
    plan = ex.a2a_plan(np.ones(cp * L, dtype=np.int64), None, cp)
    assert plan["s_first"].tolist() == [0, 0, 0, 0]
    assert plan["real_end"].tolist() == [8, 16, 24, 32]
    assert plan["back"].tolist() == [0, 8, 16, 24]
    assert plan["use_halo"] is False and plan["halo_size"] == 24
    # rank r receives every earlier chunk whole and its own
    assert plan["splits"].tolist() == [[8, 8, 8, 8], [0, 8, 8, 8], [0, 0, 8, 8], [0, 0, 0, 8]]
    assert plan["send_index"][0].tolist() == list(range(8)) * 4


def test_chunk_aligned_documents_need_no_exchange():
    cp, L = 3, 5
    ids = np.repeat(np.arange(1, cp + 1), L)
    plan = ex.a2a_plan(ids, None, cp)
    assert plan["s_first"].tolist() == [0, 5, 10]
    assert plan["back"].tolist() == [0, 0, 0]
    assert plan["use_halo"] is True and plan["halo_size"] == 0
    assert plan["splits"].tolist() == [[5, 0, 0], [0, 5, 0], [0, 0, 5]]


def test_two_rank_straddle_is_a_halo():
    # a document over positions 6..13 with L = 8: rank 1 needs 6, 7 from rank 0
    ids = np.array([1] * 6 + [2] * 8 + [3] * 2)
    plan = ex.a2a_plan(ids, None, 2)
    assert plan["s_first"].tolist() == [0, 6]
    assert plan["back"].tolist() == [0, 2]
    assert plan["use_halo"] is True and plan["halo_size"] == 2
    assert plan["splits"].tolist() == [[8, 2], [0, 8]]
    assert plan["send_index"][0].tolist() == list(range(8)) + [6, 7]


def test_padding_chunk_needs_nothing():
    cp, L = 3, 4
    ids = np.array([1] * 6 + [2] * 6)
    pad = np.zeros(12, dtype=np.uint8)
    pad[7:] = 1                                   # rank 1 keeps 4..6, rank 2 is all padding
    plan = ex.a2a_plan(ids, pad, cp)
    assert plan["s_first"].tolist() == [0, 0, 8]
    assert plan["real_end"].tolist() == [4, 7, 8]
    assert plan["splits"][:, 2].tolist() == [0, 0, 0]
    assert plan["splits"][:, 1].tolist() == [4, 3, 0]


@pytest.mark.parametrize("seed,B,cp,L,lo,hi,pad_tail,same", [
    (1, 1, 2, 8, 1, 6, 0, False), (2, 2, 3, 5, 2, 9, 3, False), (3, 1, 4, 16, 5, 40, 7, False),
    (4, 3, 4, 8, 1, 30, 0, True), (5, 2, 5, 6, 3, 20, 11, False), (6, 1, 6, 4, 1, 3, 0, False),
])
def test_range_is_what_the_queries_attend(seed, B, cp, L, lo, hi, pad_tail, same):
    """Block-diagonal causal attention (no window): a real query at p attends the
    keys of its own document not after p.  The needed range of rank r is the
    union over its real queries, and must be exactly [s_first_r, real_end_r)."""
    rng = np.random.default_rng(seed)
    ids, pad = _rand_ids(rng, B, cp * L, lo, hi, pad_tail, same)
    folded = ids.copy()
    if pad is not None:
        folded[pad != 0] = 0
    plan = ex.a2a_plan(ids, pad, cp)
    for r in range(cp):
        keys = set()
        for b in range(B):
            for p in range(r * L, (r + 1) * L):
                d = folded[b, p]
                if d == 0:
                    continue
                for j in range(p + 1):
                    if folded[b, j] == d:
                        keys.add(j)
        if keys:
            assert plan["s_first"][r] == min(keys)
            assert plan["real_end"][r] == max(keys) + 1
            # contiguous: every position in between is attended by some real query of some row
            assert len(keys) == max(keys) + 1 - min(keys)
        else:
            assert plan["s_first"][r] == plan["real_end"][r] == r * L
        assert plan["back"][r] == r * L - plan["s_first"][r]
    assert plan["use_halo"] == all(plan["back"][r] <= L for r in range(cp))
    # every source's pieces concatenate, in source order, into the range
    for r in range(cp):
        got = []
        for s in range(cp):
            off = int(plan["splits"][s, :r].sum())
            got += (s * L + plan["send_index"][s][off:off + plan["splits"][s, r]]).tolist()
        assert got == list(range(plan["s_first"][r], plan["real_end"][r]))


def test_halo_workload_straddle_matches_generator():
    """The block-diagonal halo workload (rank 1 of 2) builds its neighbourhood
    from the straddle of the document holding its first query; the plan's
    s_first for that rank is the same position."""
    w = wl.get(3)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    glob = wl._fill_row(rng, w.S_global, w.doc_len)
    dm = wl.make_doc_map(w)
    plan = ex.halo_plan(glob, None, w.cp_size)
    assert plan["s_first"][w.cp_rank] == dm.nb_start
    assert plan["real_end"][w.cp_rank] == w.S_global


def test_gather_closed_form_and_backward_adjoint():
    rng = np.random.default_rng(7)
    cp, L, B, C, D = 4, 6, 2, 3, 5
    ids, pad = _rand_ids(rng, B, cp * L, 2, 14, pad_tail=4)
    plan = ex.a2a_plan(ids, pad, cp)
    x = rng.standard_normal((B, C, cp * L, D))
    recv = ex.a2a_forward(x, plan)
    for r in range(cp):
        assert np.array_equal(recv[r], x[:, :, plan["s_first"][r]:plan["real_end"][r], :])
    g = [rng.standard_normal(t.shape) for t in recv]
    gx = ex.a2a_backward(g, plan, x.shape)
    lhs = sum(float(np.sum(recv[r] * g[r])) for r in range(cp))
    assert abs(lhs - float(np.sum(x * gx))) <= 1e-12 * max(1.0, abs(lhs))
    # closed form: every rank's gradient placed at its range, summed
    ref = np.zeros_like(x)
    for r in range(cp):
        ref[:, :, plan["s_first"][r]:plan["real_end"][r], :] += g[r]
    assert np.allclose(gx, ref, rtol=0, atol=1e-12)
