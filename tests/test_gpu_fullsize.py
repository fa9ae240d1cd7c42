"""All five workloads at full size, through the same C-ABI calls bench.py times,
checked against the fp64 oracle on outputs it can compute exactly one by one:

* segment builder: every array, bit-exact (the integer reference is cheap);
* O, LSE, dQ: sampled query rows (shard edges, document boundaries, random)
  for every q head of the first and last kv head -- each row depends only on
  itself;
* dK, dV: sampled keys whose attending query rows are few enough for the
  oracle, computed from exactly those rows (the sums are complete for them);
* structural zeros: every key no query attends is exactly 0 in dK and dV, and
  padding rows of O / dQ are exactly 0, over the whole tensors.
"""
import numpy as np
import pytest
import torch

from oracle import nbattn_oracle as orc
from sliding_window_attention_fold_amd import workloads as wl

from gpu_cases import assert_close, check_segments, run_gpu, say, workload_inputs

pytestmark = pytest.mark.gpu


def _sample_rows(inp, seg_ref, rng, n_rand=24):
    L = inp.L
    rows = {0, 1, L // 2, L - 2, L - 1}
    n = seg_ref["n_seg"]
    for s in range(n):
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


def _sample_keys(inp, seg_ref, b, rng, max_rows=1100):
    """Keys (with the query rows attending them) whose row sets stay small."""
    bs, p = _bands(inp, seg_ref, b)
    real = bs <= p
    S, L = inp.S, inp.L
    cand = []
    # the last keys of the neighbourhood, then keys spread over the covered range
    for j in list(range(S - 1, max(S - 40, -1), -7)) + rng.integers(0, S, 400).tolist():
        att = np.nonzero(real & (bs <= j) & (j <= p))[0]
        if 0 < len(att) <= max_rows:
            cand.append((int(j), att))
        if len(cand) >= 12:
            break
    keys = np.array(sorted({j for j, _ in cand}), dtype=np.int64)
    rows = np.unique(np.concatenate([a for _, a in cand])) if cand else np.zeros(0, dtype=np.int64)
    return keys, rows


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_workload(cfg):
    w = wl.get(cfg)
    inp = workload_inputs(w, "bf16")
    say(f"[full] config {cfg}: {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L={w.L} S={inp.S} W={w.window}")
    seg, out, lse, res = run_gpu(inp)
    check_segments(seg, inp)
    seg_ref = orc.segments_reference(inp.folded, inp.L, inp.window)
    rng = np.random.default_rng(1000 + cfg)
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

    b = inp.folded.shape[0] - 1          # last batch row (config 5 has four)
    for kv in sorted({0, w.Hkv - 1}):
        heads = list(range(kv * w.g, (kv + 1) * w.g))
        rows = _sample_rows(inp, seg_ref, rng)
        sl = slice(b, b + 1)
        O, LSE = orc.attention_forward(inp.q[sl], inp.k[sl], inp.v[sl], inp.folded[sl], w.window, scale,
                                       heads=heads, rows=rows)
        assert_close(f"O kv{kv}", o_np[sl][:, heads][:, :, rows], O, "bf16")
        assert_close(f"LSE kv{kv}", lse_np[sl][:, heads][:, :, rows], LSE, "bf16")
        dQ, _, _ = orc.attention_backward(inp.q[sl], inp.k[sl], inp.v[sl], inp.do[sl], inp.folded[sl], w.window,
                                          scale, kv_heads=[kv], rows=rows, keys=np.zeros(0, dtype=np.int64))
        assert_close(f"dQ kv{kv}", dq_np[sl][:, heads][:, :, rows], dQ[:, heads][:, :, rows], "bf16")
        keys, krows = _sample_keys(inp, seg_ref, b, rng)
        say(f"[full] config {cfg} kv {kv}: {len(rows)} rows, {len(keys)} keys from {len(krows)} rows")
        if len(keys):
            _, dK, dV = orc.attention_backward(inp.q[sl], inp.k[sl], inp.v[sl], inp.do[sl], inp.folded[sl],
                                               w.window, scale, kv_heads=[kv], rows=krows, keys=keys)
            assert_close(f"dK kv{kv}", dk_np[sl][:, kv][:, keys], dK[:, kv][:, keys], "bf16")
            assert_close(f"dV kv{kv}", dv_np[sl][:, kv][:, keys], dV[:, kv][:, keys], "bf16")
    # owner flags against the oracle's coverage
    for o, rank in enumerate(inp.owners):
        a, e = inp.owner_off[o], inp.owner_off[o + 1]
        assert res.attended[rank] == bool(att[:, a:e].any())
    torch.cuda.synchronize()
