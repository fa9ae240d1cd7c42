"""HIP path vs the fp64 oracle, every element, at sizes the oracle finishes in
seconds (several tiles and ragged tails), plus the edge cases of the method."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import nbattn_oracle as orc
import sliding_window_attention_fold_amd as nb
from sliding_window_attention_fold_amd import _lib
from sliding_window_attention_fold_amd import workloads as wl

from gpu_cases import assert_close, custom_inputs, full_parity, run_gpu, say, workload_inputs

pytestmark = pytest.mark.gpu

# Scaled-down versions of the five workloads (same document laws, heads ratio, head dim, window role).
SMALL = {
    "w1": wl.get(1),
    "w2s": wl.Workload(2, "small ring", B=1, Hq=4, Hkv=2, D=256, L=320, S_global=1280, q_start=960,
                       window=100, doc_len=("geometric", 1 / 160, 8, 1280), pad_tail=0, mode="ring",
                       cp_rank=3, cp_size=4),
    "w2s_d64": wl.Workload(2, "small d64", B=1, Hq=4, Hkv=2, D=64, L=320, S_global=1280, q_start=960,
                           window=100, doc_len=("geometric", 1 / 160, 8, 1280), pad_tail=0, mode="ring",
                           cp_rank=3, cp_size=4),
    "w3s": wl.Workload(3, "small halo", B=1, Hq=4, Hkv=1, D=128, L=300, S_global=600, q_start=300, window=-1,
                       doc_len=("lognormal", 4.6, 1.0, 4, 300), pad_tail=0, mode="halo", cp_rank=1, cp_size=2),
    "w4s": wl.Workload(4, "small single doc", B=1, Hq=8, Hkv=2, D=128, L=200, S_global=800, q_start=600,
                       window=-1, doc_len=("single",), pad_tail=0, mode="needed", cp_rank=3, cp_size=4),
    "w5s": wl.Workload(5, "small batched pad", B=3, Hq=4, Hkv=2, D=128, L=192, S_global=384, q_start=192,
                       window=40, doc_len=("uniform", 3, 40), pad_tail=57, mode="ring", cp_rank=1, cp_size=2,
                       outliers=True, per_row_docs=True),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads(name, dtype):
    w = SMALL[name]
    say(f"[parity] {name} {dtype} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L={w.L} W={w.window}")
    full_parity(workload_inputs(w, dtype), dtype)


def _docs(rng, S, lo, hi):
    ids = np.zeros(S, dtype=np.int32)
    pos, d = 0, 1
    while pos < S:
        n = int(rng.integers(lo, hi + 1))
        ids[pos:pos + n] = d
        pos, d = pos + n, d + 1
    return ids


EDGE = {
    # L = S: empty halo, one document, no window (plain causal attention)
    "empty_halo": lambda: dict(ids=np.ones((1, 200)), L=200, W=-1),
    # documents of length 1: every row attends only itself
    "len1_docs": lambda: dict(ids=np.arange(1, 151)[None], L=100, W=-1),
    "window0": lambda: dict(ids=_docs(np.random.default_rng(1), 260, 5, 70)[None], L=130, W=0),
    "window_ge_S": lambda: dict(ids=_docs(np.random.default_rng(2), 260, 5, 70)[None], L=130, W=1000),
    "L1": lambda: dict(ids=_docs(np.random.default_rng(3), 97, 5, 40)[None], L=1, W=-1),
    "tile_edges": lambda: dict(ids=np.repeat(np.arange(1, 9), [64, 128, 64, 64, 32, 128, 64, 64])[None], L=256,
                               W=-1),
    "mid_pad_and_negative": lambda: dict(
        ids=np.concatenate([np.full(70, 1), np.full(30, 2), np.zeros(25), np.full(40, 3), np.full(10, -4),
                            np.full(45, 5)])[None], L=150, W=50),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name, dtype):
    e = EDGE[name]()
    ids = np.asarray(e["ids"], dtype=np.int32)
    say(f"[edge] {name} {dtype} S={ids.shape[1]} L={e['L']} W={e['W']}")
    full_parity(custom_inputs(ids, None, 4, 2, 64, e["L"], e["W"], dtype, seed=11), dtype)


@pytest.mark.parametrize("hkv", [8, 2, 1])
def test_gqa_groups(hkv):
    rng = np.random.default_rng(5)
    ids = _docs(rng, 300, 10, 120)[None]
    say(f"[gqa] Hq=8 Hkv={hkv}")
    full_parity(custom_inputs(ids, None, 8, hkv, 128, 170, 60, "bf16", seed=12), "bf16")


def test_all_pad_batch_row_and_pad_mask():
    rng = np.random.default_rng(6)
    ids = np.stack([_docs(rng, 200, 10, 60), _docs(rng, 200, 10, 60)])
    pad = np.zeros_like(ids, dtype=np.uint8)
    pad[1, :] = 1           # the whole second row is padding
    pad[0, 180:] = 1        # pad tail on the first row
    say("[edge] all-pad batch row")
    inp = custom_inputs(ids, pad, 4, 2, 128, 120, 30, "bf16", seed=13, owner_off=[0, 80, 200])
    full_parity(inp, "bf16")
    seg, out, lse, res = run_gpu(inp)
    assert (out[1].float() == 0).all() and torch.isneginf(lse[1]).all()
    assert (res.dq[1].float() == 0).all() and (res.dk[1].float() == 0).all() and (res.dv[1].float() == 0).all()


def test_nothing_attended_anywhere():
    """n_seg = 0: every row is padding; all outputs zero, LSE -inf, no owner attended."""
    ids = np.ones((1, 128), dtype=np.int32)
    pad = np.ones((1, 128), dtype=np.uint8)
    say("[edge] empty shard")
    inp = custom_inputs(ids, pad, 2, 1, 64, 64, -1, "bf16", seed=14, owner_off=[0, 64, 128])
    seg, out, lse, res = run_gpu(inp)
    assert seg.header_host()["n_seg"] == 0
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    assert (res.dq.float() == 0).all() and (res.dk.float() == 0).all() and (res.dv.float() == 0).all()
    assert not any(res.attended.values())


def test_split_document_sets_status():
    """An id in two separate runs of one row violates the per-document contract: status bit 0."""
    ids = np.array([[3, 3, 0, 3, 3, 1, 1, 0]], dtype=np.int32)
    say("[builder] split document status")
    seg = nb.segment_build(torch.from_numpy(ids).cuda(), 4, -1)
    h = seg.header_host()
    ref = orc.segments_reference(ids, 4, -1)
    assert h["status"] == 1 == ref["status"]
    assert h["n_seg"] == ref["n_seg"]
    assert seg.cu_q.cpu().numpy()[:3].tolist() == ref["cu_q"].tolist()


def test_builder_random_maps():
    rng = np.random.default_rng(7)
    for trial in range(12):
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 20000))
        L = int(rng.integers(1, S + 1))
        W = int(rng.choice([-1, 0, 3, 100, 5000]))
        hi = int(rng.choice([1, 4, 50, 3000]))
        ids = np.stack([_docs(rng, S, 1, hi) for _ in range(B)])
        pad = (rng.random((B, S)) < 0.02).astype(np.uint8) if trial % 3 == 0 else None
        say(f"[builder] trial {trial} B={B} S={S} L={L} W={W}")
        seg = nb.segment_build(torch.from_numpy(ids).cuda(), L, W,
                               None if pad is None else torch.from_numpy(pad).cuda())
        folded = orc.fold_pad(ids, pad)
        ref = orc.segments_reference(folded, L, W)
        h = seg.header_host()
        n = ref["n_seg"]
        assert (h["n_seg"], h["max_q"], h["max_k"], h["status"]) == (n, ref["max_q"], ref["max_k"], ref["status"])
        assert np.array_equal(seg.folded.cpu().numpy(), folded)
        for key, m in (("cu_q", n + 1), ("cu_k", n + 1), ("q_row0", n), ("k_row0", n)):
            assert np.array_equal(getattr(seg, key).cpu().numpy()[:m], ref[key][:m]), key
        for key in ("row_seg", "row_klo", "kcov_lo"):
            assert np.array_equal(getattr(seg, key).cpu().numpy(), ref[key]), key


def test_deterministic_bitwise():
    w = SMALL["w5s"]
    inp = workload_inputs(w, "bf16")
    say("[determinism] w5s twice")
    a = run_gpu(inp)
    b = run_gpu(inp)
    for x, y in ((a[1], b[1]), (a[2], b[2]), (a[3].dq, b[3].dq), (a[3].dk, b[3].dk), (a[3].dv, b[3].dv)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["w2s", "w5s"])
def test_backward_entry_points_agree(name):
    """nb_attn_bwd, prep + main, and dq + dkdv called separately (twice, so a
    reused workspace is covered) give bit-identical dQ, dK, dV on the plain
    workspace; with the windowed workspace (stored dS, dQ = dS K) nb_attn_bwd
    and prep + main agree bit for bit, dK and dV equal the plain path's bit for
    bit and dQ agrees within the bf16 tolerance (the stored path rounds the
    same dS to bf16, from S and dP accumulated in another order)."""

    w = SMALL[name]
    inp = workload_inputs(w, "bf16")
    say(f"[entry points] {name}")
    seg, out, lse, res = run_gpu(inp)
    dev = torch.device("cuda:0")
    lib = _lib.load()
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    _, saved = nb.attn_fwd(q, k, v, seg)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    sc = D ** -0.5
    W = inp.window
    wsb_plain = lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, _lib.NB_BF16)
    wsb_win = lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S, D, _lib.NB_BF16, W)
    assert (wsb_win > wsb_plain) == (W >= 0 and D == 256)   # the stored-dS form is used at D = 256
    off_c = (ctypes.c_int32 * 2)(0, S)
    att = torch.empty((1,), dtype=torch.uint8, device=dev)

    def full(wsb):
        ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
        g = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        _lib.check(lib.nb_attn_bwd(P(do), P(q), P(k), P(v), P(saved.out), P(saved.out_resid), P(saved.lse),
                                   P(seg.buf), P(seg.folded), B, Hq, Hkv, L, S, D, sc, W, _lib.NB_BF16, P(g[0]),
                                   P(g[1]), P(g[2]), ctypes.cast(off_c, ctypes.c_void_p), 1, P(att), P(ws), wsb, sp),
                   "nb_attn_bwd")
        return g

    def prep_main(wsb, ws):
        g = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        _lib.check(lib.nb_attn_bwd_prep(P(do), P(saved.out), P(saved.out_resid), P(seg.buf), B, Hq, Hkv, L, S, D, W,
                                        _lib.NB_BF16, P(ws), wsb, sp), "prep")
        _lib.check(lib.nb_attn_bwd_main(P(do), P(q), P(k), P(v), P(saved.lse), P(seg.buf), B, Hq, Hkv, L, S, D, sc,
                                        W, _lib.NB_BF16, P(g[0]), P(g[1]), P(g[2]), P(ws), wsb, sp), "main")
        return g

    plain = full(wsb_plain)
    win = full(wsb_win)
    for x, y in zip(win, (res.dq, res.dk, res.dv)):      # the Python binding takes the windowed workspace
        assert torch.equal(x, y)
    assert torch.equal(win[1], plain[1]) and torch.equal(win[2], plain[2])
    assert_close("dQ stored-dS vs recompute", win[0].float().cpu().numpy(), plain[0].float().cpu().numpy(), "bf16")
    ws_p = torch.empty((wsb_plain,), dtype=torch.uint8, device=dev)
    ws_w = torch.empty((wsb_win,), dtype=torch.uint8, device=dev)
    for rep in range(2):
        a = prep_main(wsb_plain, ws_p)
        bw = prep_main(wsb_win, ws_w)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, plain)), f"prep+main plain {rep}"
        assert all(torch.equal(x, y) for x, y in zip(bw, win)), f"prep+main windowed {rep}"
        dq2 = torch.full_like(q, float("nan"))
        dk2 = torch.full_like(k, float("nan"))
        dv2 = torch.full_like(v, float("nan"))
        _lib.check(lib.nb_attn_bwd_dq(P(do), P(q), P(k), P(v), P(saved.out), P(saved.out_resid), P(saved.lse),
                                      P(seg.buf), B, Hq, Hkv, L, S, D, sc, W, _lib.NB_BF16, P(dq2), P(ws_p), wsb_plain,
                                      sp), "dq")
        _lib.check(lib.nb_attn_bwd_dkdv(P(do), P(q), P(k), P(v), P(saved.lse), P(seg.buf), B, Hq, Hkv, L, S, D, sc,
                                        W, _lib.NB_BF16, P(dk2), P(dv2), P(ws_p), wsb_plain, sp), "dkdv")
        torch.cuda.synchronize()
        assert torch.equal(dq2, plain[0]) and torch.equal(dk2, plain[1]) and torch.equal(dv2, plain[2]), \
            f"dq+dkdv {rep}"


def test_autograd_function_matches_direct_calls():
    w = SMALL["w2s"]
    inp = workload_inputs(w, "bf16")
    say("[autograd] w2s")
    dev = torch.device("cuda:0")
    seg = nb.segment_build(torch.from_numpy(inp.ids).to(dev), inp.L, inp.window)
    q, k, v, do = (t.to(dev).clone().requires_grad_(True) for t in (inp.q, inp.k, inp.v, inp.do))
    out = nb.neighbourhood_attention(q, k, v, seg)
    out.backward(do.detach())
    ref_out, saved = nb.attn_fwd(q.detach(), k.detach(), v.detach(), seg)
    r = nb.attn_bwd(saved, do.detach())
    assert torch.equal(out.detach(), ref_out)
    assert torch.equal(q.grad, r.dq) and torch.equal(k.grad, r.dk) and torch.equal(v.grad, r.dv)


def test_dropout_rejected_before_launch():
    inp = workload_inputs(SMALL["w1"], "bf16")
    dev = torch.device("cuda:0")
    seg = nb.segment_build(torch.from_numpy(inp.ids).to(dev), inp.L, inp.window)
    with pytest.raises(_lib.NbError) as ei:
        nb.attn_fwd(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), seg, dropout_p=0.1)
    assert ei.value.status == _lib.NB_ERR_UNSUPPORTED


def test_owner_dict_wrapped_owners_are_zero():
    """_owner_grad_dict: rank 1 of 4 with n_prior = 3 also returns the wrapped owners 3 and 2, as zeros."""
    rng = np.random.default_rng(8)
    ids = _docs(rng, 256, 20, 90)[None]
    inp = custom_inputs(ids, None, 2, 1, 64, 128, 64, "bf16", seed=15, owner_off=[0, 128, 256])
    dev = torch.device("cuda:0")
    seg = nb.segment_build(torch.from_numpy(inp.ids).to(dev), inp.L, inp.window)
    _, saved = nb.attn_fwd(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), seg)
    r = nb.attn_bwd(saved, inp.do.to(dev), nb.OwnerTable([0, 128, 256], [0, 1], cp_rank=1, cp_size=4, n_prior=3))
    assert sorted(r.dk_by_owner) == [0, 1, 2, 3]
    for o in (2, 3):
        assert r.dk_by_owner[o].shape == (1, 1, 128, 64) and (r.dk_by_owner[o].float() == 0).all()
        assert not r.attended[o]


STORED_DS_CASES = [  # seed, B, Hq, Hkv, L, S, window, doc lengths lo..hi, pad tail, dtype
    (31, 1, 2, 1, 97, 333, 0, 5, 60, 0, "bf16"),      # window 0: the diagonal only
    (32, 2, 4, 2, 130, 161, 1, 1, 40, 7, "bf16"),     # window 1, two batch rows, padding tail
    (33, 1, 4, 1, 200, 515, 33, 20, 300, 0, "bf16"),  # GQA 4, keys not a multiple of 32
    (34, 2, 2, 2, 64, 64, 100, 10, 50, 3, "f32"),     # window wider than the neighbourhood
    (35, 1, 2, 1, 257, 1100, 700, 100, 900, 31, "bf16"),
    (36, 1, 2, 1, 100, 5000, 4096, 200, 3000, 0, "bf16"),   # the widest window with a dS buffer
    (37, 1, 2, 1, 64, 4300, 4097, 100, 2000, 5, "bf16"),    # one wider: the recompute form on the same calls
]


@pytest.mark.parametrize("case", STORED_DS_CASES)
def test_stored_ds_backward_edges(case):
    """The stored-dS backward (D = 256 with a window) at ragged sizes: against the
    oracle element by element, and against the recompute form (dK, dV bit-identical,
    dQ within tolerance)."""
    seed, B, Hq, Hkv, L, S, W, lo, hi, pt, dt = case
    rng = np.random.default_rng(seed)
    ids = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        pos, d = 0, 1
        while pos < S:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    pad = None
    if pt:
        pad = np.zeros((B, S), dtype=np.uint8)
        pad[:, S - pt:] = 1
    inp = custom_inputs(ids, pad, Hq, Hkv, 256, L, W, dt, seed)
    say(f"[stored dS] seed={seed} B={B} L={L} S={S} W={W} {dt}")
    full_parity(inp, dt)   # the Python binding takes the stored-dS workspace
    dev = torch.device("cuda:0")
    pad_d = None if pad is None else torch.from_numpy(pad).to(dev)
    seg = nb.segment_build(torch.from_numpy(ids).to(dev), L, W, pad_d)
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    _, saved = nb.attn_fwd(q, k, v, seg)
    a = nb.attn_bwd(saved, do, stored_ds=True)
    r = nb.attn_bwd(saved, do, stored_ds=False)
    assert torch.equal(a.dk, r.dk) and torch.equal(a.dv, r.dv)
    assert_close("dQ stored vs recompute", a.dq.float().cpu().numpy(), r.dq.float().cpu().numpy(), dt)
    # the workspace's old contents must not matter: filled with 0xff bytes (NaN in
    # either dtype) it gives the same bits (a dS block read but never written shows)
    lib = _lib.load()
    D, code = q.shape[3], _lib.NB_BF16 if dt == "bf16" else _lib.NB_F32
    wsb = lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S, D, code, W)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device=dev)
    g = [torch.empty_like(t) for t in (q, k, v)]
    att = torch.empty((1,), dtype=torch.uint8, device=dev)
    off_c = (ctypes.c_int32 * 2)(0, S)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _lib.check(lib.nb_attn_bwd(P(do), P(q), P(k), P(v), P(saved.out), P(saved.out_resid), P(saved.lse), P(seg.buf),
                               P(seg.folded), B, Hq, Hkv, L, S, D, saved.scale, W, code, P(g[0]), P(g[1]), P(g[2]),
                               ctypes.cast(off_c, ctypes.c_void_p), 1, P(att), P(ws), wsb,
                               ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)), "nb_attn_bwd")
    assert torch.equal(g[0], a.dq) and torch.equal(g[1], a.dk) and torch.equal(g[2], a.dv)


def test_training_step_never_synchronises():
    """segment_build -> attn_fwd -> attn_bwd, the autograd wrapper and the chunk-table
    calls enqueue work only: under torch's sync debug mode "error" any device-to-host
    read or stream synchronisation inside them raises (cp_local_ring page,
    _cached_sliding_segments: the point of building segments once per step is to keep
    host syncs out of the layers).  The owner flags stay on the device until read."""
    w = SMALL["w2s"]
    inp = workload_inputs(w, "bf16")
    say("[nosync] w2s")
    dev = torch.device("cuda:0")
    ids = torch.from_numpy(inp.ids).to(dev)
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    ql = q.clone().requires_grad_(True)
    kl, vl = k.clone().requires_grad_(True), v.clone().requires_grad_(True)
    off = inp.owner_off
    k_chunks = [k[:, :, off[c]:off[c + 1]].contiguous() for c in range(len(off) - 1)]
    v_chunks = [v[:, :, off[c]:off[c + 1]].contiguous() for c in range(len(off) - 1)]
    table = nb.OwnerTable(off, inp.owners, inp.cp_rank, inp.cp_size)
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        seg = nb.segment_build(ids, inp.L, inp.window)
        _, saved = nb.attn_fwd(q, k, v, seg)
        res = nb.attn_bwd(saved, do, table)
        out = nb.neighbourhood_attention(ql, kl, vl, seg)
        out.backward(do)
        chunks = nb.ring_window_chunks(k_chunks, v_chunks, inp.window)
        seg2 = nb.segment_build(ids[:, inp.S - sum(c.length for c in chunks):].contiguous(), inp.L, inp.window)
        _, saved_c = nb.attn_fwd_chunks(q, chunks, seg2)
        dq_c, dks, dvs, att_c = nb.attn_bwd_chunks(saved_c, do)
    finally:
        torch.cuda.set_sync_debug_mode("default")
    torch.cuda.synchronize()
    # the flags are read (and only now synchronised) after the step
    ref = orc.key_attended(inp.folded, inp.L, inp.window)
    for o, rank in enumerate(inp.owners):
        assert res.attended[rank] == bool(ref[:, off[o]:off[o + 1]].any())
    assert torch.equal(ql.grad, res.dq) and torch.equal(kl.grad, res.dk)
    assert_close("dQ chunks", dq_c.float().cpu().numpy(), res.dq.float().cpu().numpy(), "bf16")
    for c in range(len(chunks)):
        assert att_c[c] == bool(dks[c].any() or dvs[c].any())


@pytest.mark.parametrize("name", ["w2s", "w2s_d64", "w5s"])
def test_output_residual_codes_and_delta(name):
    """The forward's byte residual of O (include/nbattn.h, o_resid): every code in [-127, 127]; the decoded residual
    (code / 254 of the bf16 value's ulp) moves O toward the fp64 oracle's O; and the prep's Delta, dO . (O +
    decoded residual) on every real row and 0 on the others, equals the same sum formed on the host in fp64 from the
    header's definition.  The kernel's fp32 O is itself about as far from the exact O as its bf16 rounding (P is
    rounded to bf16 before P V), so the residual cannot close the whole gap: a CPU emulation of that arithmetic gives
    a median-error ratio of 0.60-0.67, a max-error ratio near 0.33 and a correlation of 0.81-0.85 between the
    residual and the oracle's correction, at 40 to 300 keys per row.  Codes of the wrong sign, scale or none at all
    fail the bounds below."""
    inp = workload_inputs(SMALL[name], "bf16")
    say(f"[residual codes] {name}")
    dev = torch.device("cuda:0")
    lib = _lib.load()
    ids = torch.from_numpy(inp.ids).to(dev)
    pad = None if inp.pad is None else torch.from_numpy(np.ascontiguousarray(inp.pad)).to(dev)
    seg = nb.segment_build(ids, inp.L, inp.window, pad)
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    out, saved = nb.attn_fwd(q, k, v, seg)
    B, Hq, L, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    wsb = lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, _lib.NB_BF16)
    ws = torch.full((wsb,), 255, dtype=torch.uint8, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _lib.check(lib.nb_attn_bwd_prep(P(do), P(out), P(saved.out_resid), P(seg.buf), B, Hq, Hkv, L, S, D, inp.window,
                                    _lib.NB_BF16, P(ws), wsb, sp), "prep")
    torch.cuda.synchronize()
    assert saved.out_resid.dtype == torch.int8 and saved.out_resid.shape == out.shape
    codes = saved.out_resid.cpu().numpy().astype(np.float64)
    assert codes.min() >= -127 and codes.max() <= 127
    o_b = out.float().cpu().numpy().astype(np.float64)
    be = (out.cpu().view(torch.int16).numpy().astype(np.int32) >> 7) & 0xFF
    ulp = np.ldexp(1.0, np.maximum(be, 1) - 134)
    o_fine = o_b + codes / 254.0 * ulp
    O, _ = orc.attention_forward(inp.q, inp.k, inp.v, inp.folded, inp.window, D ** -0.5)
    real = orc.real_rows(inp.folded, inp.L)
    rr = np.broadcast_to(real[:, None, :, None], o_b.shape)
    err_b, err_f = np.abs(o_b - O)[rr], np.abs(o_fine - O)[rr]
    assert np.median(err_f) <= 0.8 * np.median(err_b), (np.median(err_f), np.median(err_b))
    assert err_f.max() <= err_b.max()
    corr = np.corrcoef((o_fine - o_b)[rr], (O - o_b)[rr])[0, 1]
    assert corr > 0.6, corr
    delta = ws[:B * Hq * L * 4].view(torch.float32).cpu().numpy().reshape(B, Hq, L).astype(np.float64)
    want = (inp.do.double().numpy() * o_fine).sum(-1)
    want[~np.broadcast_to(real[:, None, :], want.shape)] = 0.0
    assert np.allclose(delta, want, rtol=1e-5, atol=1e-5 * np.abs(want).max())
