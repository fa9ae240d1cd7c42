"""GPU parity of the zero-copy chunk-table path (nb_attn_fwd_chunks /
nb_attn_bwd_chunks) through the C-ABI.

1. Any chunking of a neighbourhood, with chunks embedded at arbitrary rows of
   larger buffers, must give bit-identical O, LSE, dQ and chunk-row dK/dV to
   the concatenated path (the same tiles in the same order), exact zeros on the
   buffers' other rows, and the same attended flags.  The cases cover key tiles
   that straddle a chunk boundary, key ranges over three or more chunks (the
   general per-tile lookup and the deferred dQ items) and a last chunk shorter
   than a key tile.
2. The windowed ring neighbourhood trimmed to the keys the window reaches
   (ring_window_chunks) against the fp64 oracle on the full neighbourhood: the
   shard's O, LSE, dQ and the kept keys' dK/dV within tolerance, every other key
   an exact zero.
"""
import numpy as np
import pytest
import torch

from oracle import nbattn_oracle as orc
import sliding_window_attention_fold_amd as nb
from sliding_window_attention_fold_amd import workloads as wl
from gpu_cases import assert_close, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _docmap(rng, B, S, L, pad_tail=0, lo=5, hi=90):
    ids = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        pos, d = 0, 1
        while pos < S:
            n = int(rng.integers(lo, hi))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    pad = None
    if pad_tail:
        pad = np.zeros((B, S), dtype=np.uint8)
        pad[:, S - pad_tail:] = 1
    return ids, pad


CASES = [  # seed, B, Hq, Hkv, D, L, S, window, pad_tail, chunk lengths, dtype
    (1, 1, 2, 1, 64, 96, 200, 40, 0, [1, 7, 33, 63, 96], torch.bfloat16),
    (2, 2, 4, 2, 128, 130, 300, -1, 9, [100, 70, 130], torch.bfloat16),
    (3, 1, 4, 2, 256, 128, 250, 64, 0, [17, 105, 128], torch.bfloat16),
    (4, 1, 2, 1, 128, 64, 161, 50, 0, [5, 92, 64], torch.float32),
    (5, 1, 2, 2, 256, 70, 137, -1, 3, [67, 70], torch.float32),
    # long documents over short chunks: ranges touching 3+ chunks (general lookup, deferred dQ items)
    (6, 1, 4, 2, 128, 100, 200, -1, 0, [40, 20, 20, 20, 100], torch.bfloat16),
    (7, 1, 2, 1, 256, 100, 200, -1, 0, [45, 15, 20, 20, 100], torch.bfloat16),
    # the last chunk shorter than a key tile: the tile holding the boundary would run past it
    (8, 1, 2, 1, 128, 10, 160, -1, 0, [150, 10], torch.bfloat16),
    (9, 1, 2, 1, 256, 20, 163, 60, 0, [143, 20], torch.bfloat16),
    # windowed at D = 256 (the stored-dS form): a dQ workgroup's keys over five chunks, and fp32
    (10, 1, 2, 1, 256, 128, 250, 100, 5, [30, 40, 30, 20, 130], torch.bfloat16),
    (11, 1, 2, 2, 256, 96, 200, 50, 0, [60, 44, 96], torch.float32),
]


@pytest.mark.parametrize("case", CASES)
def test_chunks_match_concatenated_bitwise(case):
    seed, B, Hq, Hkv, D, L, S, W, pad_tail, lens, dt = case
    assert sum(lens) == S
    say(f"[chunks] case seed={seed} D={D} S={S} chunks={lens} {dt}")
    rng = np.random.default_rng(seed)
    ids, pad = _docmap(rng, B, S, L, pad_tail, *((60, 160) if W < 0 and len(lens) > 3 else (5, 90)))
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, Hq, L, D), generator=g).to(dt).to(DEV)
    k = torch.randn((B, Hkv, S, D), generator=g).to(dt).to(DEV)
    v = torch.randn((B, Hkv, S, D), generator=g).to(dt).to(DEV)
    do = torch.randn((B, Hq, L, D), generator=g).to(dt).to(DEV)
    seg = nb.segment_build(torch.from_numpy(ids).to(DEV), L, W,
                           None if pad is None else torch.from_numpy(pad).to(DEV))
    out, saved = nb.attn_fwd(q, k, v, seg)
    offs = np.concatenate([[0], np.cumsum(lens)]).tolist()
    owners = nb.OwnerTable(offs, list(range(len(lens))))
    # the same keys embedded at random rows of larger chunk buffers
    chunks = []
    for c, n in enumerate(lens):
        extra_lo, extra_hi = int(rng.integers(0, 20)), int(rng.integers(0, 20))
        kb = torch.randn((B, Hkv, extra_lo + n + extra_hi, D), generator=g).to(dt).to(DEV)
        vb = torch.randn((B, Hkv, extra_lo + n + extra_hi, D), generator=g).to(dt).to(DEV)
        kb[:, :, extra_lo:extra_lo + n] = k[:, :, offs[c]:offs[c + 1]]
        vb[:, :, extra_lo:extra_lo + n] = v[:, :, offs[c]:offs[c + 1]]
        chunks.append(nb.KvChunk(kb, vb, extra_lo, n))
    out_c, saved_c = nb.attn_fwd_chunks(q, chunks, seg)
    assert torch.equal(out_c, out)
    assert torch.equal(saved_c.lse, saved.lse)
    # both backward forms (dQ from stored dS with a window at D = 256, else the
    # recompute) against the same form over the concatenated neighbourhood
    for stored in (False, True):
        ref = nb.attn_bwd(saved, do, owners, stored_ds=stored)
        dq, dks, dvs, att = nb.attn_bwd_chunks(saved_c, do, stored_ds=stored)
        assert torch.equal(dq, ref.dq)
        for c, ch in enumerate(chunks):
            lo, hi = ch.start, ch.start + ch.length
            assert torch.equal(dks[c][:, :, lo:hi], ref.dk[:, :, offs[c]:offs[c + 1]])
            assert torch.equal(dvs[c][:, :, lo:hi], ref.dv[:, :, offs[c]:offs[c + 1]])
            assert not dks[c][:, :, :lo].any() and not dks[c][:, :, hi:].any()
            assert not dvs[c][:, :, :lo].any() and not dvs[c][:, :, hi:].any()
            assert att[c] == ref.attended[c]


@pytest.mark.parametrize("cfg", [1, 2])
def test_window_trimmed_ring_matches_oracle(cfg):
    """The ring workloads at a size the oracle finishes in seconds: the rank's
    prior chunks reduced to the last W keys, read in place."""
    w = wl.get(cfg)
    if cfg == 2:
        w = wl.small_variant(w, L=256, S_global=1024, q_start=768, window=100, Hq=4, Hkv=2)
    dm = wl.make_doc_map(w)
    q, k, v, do = wl.make_tensors(w, dm.S, "bf16")
    L, S, W, C = w.L, dm.S, w.window, len(dm.owner_off) - 1
    say(f"[chunks] trimmed ring config {cfg}: L={L} S={S} W={W} chunks={C}")
    folded = orc.fold_pad(dm.doc_ids, dm.pad_mask)
    o_ref, lse_ref = orc.attention_forward(q, k, v, folded, W, w.D ** -0.5)
    dq_ref, dk_ref, dv_ref = orc.attention_backward(q, k, v, do, folded, W, w.D ** -0.5)
    kd, vd = k.to(DEV), v.to(DEV)
    k_chunks = [kd[:, :, dm.owner_off[c]:dm.owner_off[c + 1]].contiguous() for c in range(C)]
    v_chunks = [vd[:, :, dm.owner_off[c]:dm.owner_off[c + 1]].contiguous() for c in range(C)]
    chunks = nb.ring_window_chunks(k_chunks, v_chunks, W)
    S2 = sum(c.length for c in chunks)
    nb0 = S - S2                                  # first key of the trimmed neighbourhood
    ids2 = torch.from_numpy(np.ascontiguousarray(dm.doc_ids[:, nb0:])).to(DEV)
    pad2 = None if dm.pad_mask is None else torch.from_numpy(np.ascontiguousarray(dm.pad_mask[:, nb0:])).to(DEV)
    seg = nb.segment_build(ids2, L, W, pad2)
    out, saved = nb.attn_fwd_chunks(q.to(DEV), chunks, seg)
    dq, dks, dvs, att = nb.attn_bwd_chunks(saved, do.to(DEV))
    assert_close("O", out.float().cpu().numpy(), o_ref, "bf16")
    assert_close("LSE", saved.lse.cpu().numpy(), lse_ref, "bf16")
    assert_close("dQ", dq.float().cpu().numpy(), dq_ref, "bf16")
    # whole chunk-gradient buffers against the oracle's full-neighbourhood dK/dV
    full_dk = np.zeros_like(dk_ref)
    full_dv = np.zeros_like(dv_ref)
    first_chunk = C - len(chunks)
    for i, ch in enumerate(chunks):
        c = first_chunk + i
        full_dk[:, :, dm.owner_off[c]:dm.owner_off[c + 1]] = dks[i].float().cpu().numpy()
        full_dv[:, :, dm.owner_off[c]:dm.owner_off[c + 1]] = dvs[i].float().cpu().numpy()
    assert_close("dK", full_dk, dk_ref, "bf16")
    assert_close("dV", full_dv, dv_ref, "bf16")
    assert not full_dk[:, :, :nb0].any() and not full_dv[:, :, :nb0].any()
