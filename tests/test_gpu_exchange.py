"""GPU parity of the exchange planners and the emulated needed-range exchange
against the CPU oracle (oracle/exchange_oracle.py), through the C-ABI.

Integer outputs (plan, send_index) and the gather (a copy) must be bit-exact;
the backward sums in fp32 and rounds once, so it is checked against the fp64
oracle within one rounding of the output type."""
import numpy as np
import pytest
import torch

from oracle import exchange_oracle as ex
from sliding_window_attention_fold_amd import exchange as xg
from sliding_window_attention_fold_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _rand_ids(rng, B, N, lo, hi, pad_tail=0):
    ids = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
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


def _plan(ids, pad, P):
    print(f"[exchange] plan B={ids.shape[0]} N={ids.shape[1]} P={P}", flush=True)
    t_ids = torch.from_numpy(np.ascontiguousarray(ids)).to(DEV)
    t_pad = None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to(DEV)
    return xg.exchange_plan(t_ids, P, t_pad)


def _check_plan(gp, op):
    assert gp.L == op["L"]
    assert gp.use_halo == op["use_halo"] and gp.halo_size == op["halo_size"]
    assert gp.s_first.tolist() == op["s_first"].tolist()
    assert gp.real_end.tolist() == op["real_end"].tolist()
    assert gp.back.tolist() == op["back"].tolist()
    assert np.array_equal(gp.splits, op["splits"])
    assert gp.total == int((op["real_end"] - op["s_first"]).sum())
    si = xg.send_index(gp)
    for s in range(len(si)):
        assert si[s].cpu().numpy().tolist() == op["send_index"][s].tolist()


CASES = [  # seed, B, P, L, lo, hi, pad_tail
    (11, 1, 1, 64, 3, 40, 0), (12, 1, 2, 40, 1, 9, 5), (13, 2, 4, 24, 2, 60, 7), (14, 3, 8, 16, 1, 100, 0),
    (15, 1, 5, 33, 30, 200, 0), (16, 2, 64, 2, 1, 5, 3), (17, 1, 3, 50, 200, 400, 0), (18, 4, 6, 10, 1, 3, 60),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_plan_gather_scatter_match_oracle(case, dtype):
    seed, B, P, L, lo, hi, pad_tail = case
    rng = np.random.default_rng(seed)
    ids, pad = _rand_ids(rng, B, P * L, lo, hi, pad_tail)
    op = ex.a2a_plan(ids, pad, P)
    gp = _plan(ids, pad, P)
    _check_plan(gp, op)
    C, D = 3, 16
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn((B, C, P * L, D), generator=g).to(dtype)
    recv = xg.needed_gather(x.to(DEV), gp)
    ref = ex.a2a_forward(x.double().numpy(), op)
    for r in range(P):
        assert np.array_equal(recv[r].cpu().double().numpy(), ref[r]), r
    grads = [torch.randn(t.shape, generator=g).to(dtype) for t in ref]
    got = xg.needed_scatter_add([t.to(DEV) for t in grads], gp, B, C, D, dtype, DEV).cpu().double().numpy()
    want = ex.a2a_backward([t.double().numpy() for t in grads], op, x.shape)
    mag = ex.a2a_backward([np.abs(t.double().numpy()) for t in grads], op, x.shape)
    # one rounding to the output type, plus fp32 accumulation over at most P terms
    rnd = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -23
    assert np.all(np.abs(got - want) <= rnd * np.abs(want) + P * 2.0 ** -23 * mag)
    untouched = np.ones(P * L, dtype=bool)
    for r in range(P):
        untouched[op["s_first"][r]:op["real_end"][r]] = False
    assert np.all(got[:, :, untouched, :] == 0)


def test_single_document_and_all_padding():
    ids = np.ones((1, 8 * 4), dtype=np.int32)
    _check_plan(_plan(ids, None, 8), ex.a2a_plan(ids, None, 8))
    pad = np.ones((2, 12), dtype=np.uint8)
    ids2 = np.ones((2, 12), dtype=np.int32)
    gp = _plan(ids2, pad, 3)
    _check_plan(gp, ex.a2a_plan(ids2, pad, 3))
    assert gp.total == 0 and gp.splits.sum() == 0 and gp.use_halo


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_plans_full_size(cfg):
    """The workloads' global doc maps at their real size and world: the plan and
    send_index bit-exact; the gather against its closed form (rank r receives
    x[:, :, s_first_r:real_end_r]) and the backward against the sum of the
    ranks' gradients placed at their ranges (an independent torch sum)."""
    w = wl.get(cfg)
    ids, pad = wl.global_doc_map(w)
    op = ex.a2a_plan(ids, pad, w.cp_size)
    gp = _plan(ids, pad, w.cp_size)
    _check_plan(gp, op)
    B, C, D = ids.shape[0], 2, 64
    g = torch.Generator("cpu").manual_seed(cfg)
    x = torch.randn((B, C, ids.shape[1], D), generator=g).to(torch.bfloat16).to(DEV)
    recv = xg.needed_gather(x, gp)
    for r in range(w.cp_size):
        assert torch.equal(recv[r], x[:, :, int(gp.s_first[r]):int(gp.real_end[r])])
    grads = [torch.randn(t.shape, generator=g).to(torch.bfloat16).to(DEV) for t in recv]
    got = xg.needed_scatter_add(grads, gp, B, C, D, torch.bfloat16, DEV).float()
    want = torch.zeros_like(got)
    for r in range(w.cp_size):
        want[:, :, int(gp.s_first[r]):int(gp.real_end[r])] += grads[r].float()
    assert torch.all((got - want).abs() <= 2.0 ** -8 * want.abs() + 1e-6)


def test_autograd_function_backward_is_the_index_add():
    rng = np.random.default_rng(3)
    ids, pad = _rand_ids(rng, 1, 4 * 32, 5, 70)
    gp = _plan(ids, pad, 4)
    x = torch.randn((1, 2, 128, 32), device=DEV, dtype=torch.float32, requires_grad=True)
    outs = xg.needed_kv_exchange(x, gp)
    weights = [torch.randn_like(o) for o in outs]
    sum((o * wt).sum() for o, wt in zip(outs, weights)).backward()
    want = xg.needed_scatter_add(weights, gp, 1, 2, 32, torch.float32, DEV)
    assert torch.allclose(x.grad, want, rtol=1e-6, atol=1e-6)
