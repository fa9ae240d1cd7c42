"""nb_attn_bwd_noalloc (the backward for callers that cannot allocate) against
nb_attn_bwd with a caller workspace of nb_attn_bwd_workspace_bytes, through the
C-ABI: the two share their kernels and work orders, so dQ, dK, dV and the owner
flags must be bit-identical.  Two calls in a row, the second on a smaller input,
so the static workspace is reused with different contents."""
import ctypes

import numpy as np
import pytest
import torch

from sliding_window_attention_fold_amd import _lib
import sliding_window_attention_fold_amd as nb

from gpu_cases import custom_inputs, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731


def _docs(rng, B, S, lo, hi):
    ids = np.zeros((B, S), dtype=np.int32)
    for b in range(B):
        pos, d = 0, 1
        while pos < S:
            n = int(rng.integers(lo, hi + 1))
            ids[b, pos:pos + n] = d
            pos, d = pos + n, d + 1
    return ids


def _both(lib, inp, D, dtype):
    seg = nb.segment_build(torch.from_numpy(inp.ids).to(DEV), inp.L, inp.window)
    q, k, v, do = (t.to(DEV).contiguous() for t in (inp.q, inp.k, inp.v, inp.do))
    out, saved = nb.attn_fwd(q, k, v, seg)
    B, Hq, L, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    dt = _lib.NB_BF16 if dtype == "bf16" else _lib.NB_F32
    off = inp.owner_off
    n_owner = len(off) - 1
    off_c = (ctypes.c_int32 * len(off))(*off)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    res = []
    for mode in ("workspace", "noalloc"):
        dq = torch.full_like(q, float("nan"))
        dk = torch.full_like(k, float("nan"))
        dv = torch.full_like(v, float("nan"))
        att = torch.full((n_owner,), 7, dtype=torch.uint8, device=DEV)
        common = (P(do), P(q), P(k), P(v), P(out), P(saved.out_resid), P(saved.lse), P(seg.buf), P(seg.folded),
                  B, Hq, Hkv, L, S, D, saved.scale, seg.window, dt, P(dq), P(dk), P(dv),
                  ctypes.cast(off_c, ctypes.c_void_p), n_owner, P(att))
        if mode == "workspace":
            ws_bytes = lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dt)
            ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=DEV)
            st = lib.nb_attn_bwd(*common, P(ws), ws_bytes, stream)
        else:
            st = lib.nb_attn_bwd_noalloc(*common, stream)
        assert st == _lib.NB_OK, (mode, _lib.status_string(st))
        torch.cuda.synchronize()
        res.append((dq, dk, dv, att))
    for a, b_ in zip(res[0], res[1]):
        assert torch.equal(a, b_)
    assert not torch.isnan(res[1][0].float()).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_backward_matches_workspace_backward(dtype):
    lib = _lib.load()
    assert lib.nb_attn_bwd_noalloc_max_workspace_bytes() == 8 << 20
    rng = np.random.default_rng(71)
    # first call: two batch rows, GQA 4, D = 128, window, three owners; second: smaller, D = 64, no window
    ids1 = _docs(rng, 2, 900, 20, 400)
    inp1 = custom_inputs(ids1, None, 8, 2, 128, 500, 150, dtype, seed=72, owner_off=[0, 400, 650, 900])
    say(f"[noalloc] {dtype} call 1: B=2 Hq=8 Hkv=2 D=128 L=500 S=900 W=150")
    _both(lib, inp1, 128, dtype)
    ids2 = _docs(rng, 1, 300, 10, 120)
    inp2 = custom_inputs(ids2, None, 2, 1, 64, 130, -1, dtype, seed=73, owner_off=[0, 170, 300])
    say(f"[noalloc] {dtype} call 2: B=1 Hq=2 Hkv=1 D=64 L=130 S=300 W=-1")
    _both(lib, inp2, 64, dtype)
