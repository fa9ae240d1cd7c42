"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and its host-side preflight rejects bad arguments before launching."""
import ctypes
import os
import re

import numpy as np
import pytest

from sliding_window_attention_fold_amd import _lib
from sliding_window_attention_fold_amd import workloads as wl

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(nb_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.nb_version() == 100
    assert _lib.status_string(0) == "ok"
    for s in range(1, 6):
        assert len(_lib.status_string(s)) > 10
    assert _lib.status_string(99) == "unknown status"


def test_segment_buffer_sizes():
    lib = _lib.load()
    assert lib.nb_segment_buffer_elems(0, 1, 1) == 0
    assert lib.nb_segment_buffer_elems(1, 5, 4) == 0          # L > S
    n = lib.nb_segment_buffer_elems(2, 8, 16)
    N = 16
    assert lib.nb_segment_offset_cu_q(2, 8) == 16
    assert lib.nb_segment_offset_cu_k(2, 8) == 16 + N + 1
    assert lib.nb_segment_offset_row_klo(2, 8) == 16 + 2 * (N + 1) + 3 * N
    assert n >= lib.nb_segment_offset_kcov_lo(2, 8) + 2 + 2 * 16
    # the forward's launch order follows kcov_lo, 16-element aligned, one entry per 128-row tile
    for B, L, S in ((2, 8, 16), (3, 1000, 4000), (1, 8192, 65536)):
        fo = lib.nb_segment_offset_fwd_order(B, L)
        assert fo >= lib.nb_segment_offset_kcov_lo(B, L) + B and fo % 16 == 0
        assert lib.nb_segment_buffer_elems(B, L, S) >= fo + B * ((L + 127) // 128)


def _r256(n):
    return (n + 255) // 256 * 256


def test_backward_workspace_sizes():
    """The stored-dS room: B * Hq * round_up(L, 32) rows of round_up(span + 96, 32)
    elements (span = the window, or the chunk length for a ring chunk), 256-byte
    rounded, only at D = 256, only under 2 GiB; a window above 4096 gets none."""
    lib = _lib.load()
    bf, f32 = _lib.NB_BF16, _lib.NB_F32
    base = lib.nb_attn_bwd_workspace_bytes(2, 4, 2, 100, 300, 256, bf)
    assert base > 0
    win = lib.nb_attn_bwd_workspace_bytes_window
    assert win(2, 4, 2, 100, 300, 256, bf, 40) == base + _r256(2 * 4 * 128 * 160 * 2)   # 40 + 96 -> 160
    assert win(2, 4, 2, 100, 300, 256, f32, 40) == lib.nb_attn_bwd_workspace_bytes(2, 4, 2, 100, 300, 256, f32) \
        + _r256(2 * 4 * 128 * 160 * 4)
    assert win(2, 4, 2, 100, 300, 256, bf, 0) == base + _r256(2 * 4 * 128 * 96 * 2)
    assert win(2, 4, 2, 100, 300, 256, bf, -1) == base                 # no window
    assert win(2, 4, 2, 100, 300, 256, bf, 4097) == base               # window too wide
    assert win(2, 4, 2, 100, 300, 128, bf, 40) == lib.nb_attn_bwd_workspace_bytes(2, 4, 2, 100, 300, 128, bf)
    # over 2 GiB of dS: none (64 heads x 8192 rows x 4192 keys x 2 bytes)
    assert win(1, 64, 8, 8192, 16384, 256, bf, 4096) == lib.nb_attn_bwd_workspace_bytes(1, 64, 8, 8192, 16384, 256, bf)
    ring = lib.nb_ring_chunk_bwd_workspace_bytes
    assert ring(1, 16, 8, 4096, 4096, 256, bf) == lib.nb_attn_bwd_workspace_bytes(1, 16, 8, 4096, 4096, 256, bf) \
        + _r256(16 * 4096 * 4192 * 2)                                    # 4096 + 96 = 4192 keys per row
    assert ring(1, 2, 1, 97, 300, 64, bf) == lib.nb_attn_bwd_workspace_bytes(1, 2, 1, 97, 300, 64, bf)
    assert ring(0, 2, 1, 97, 300, 256, bf) == 0


FAKE = 0x100000  # an aligned address that is never dereferenced: every call below fails preflight


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, seg=FAKE, B=1, Hq=2, Hkv=1, L=8, S=16, D=64,
             scale=0.125, W=-1, drop=0.0, dtype=_lib.NB_BF16)
    a.update(kw)
    return _lib.load().nb_attn_fwd(a["q"], a["k"], a["v"], a["o"], None, a["lse"], a["seg"], a["B"], a["Hq"],
                                   a["Hkv"], a["L"], a["S"], a["D"], a["scale"], a["W"], a["drop"],
                                   a["dtype"], None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.NB_ERR_INVALID_ARG),
    (dict(k=FAKE + 8), _lib.NB_ERR_INVALID_ARG),          # misaligned
    (dict(Hq=3, Hkv=2), _lib.NB_ERR_INVALID_ARG),
    (dict(L=17), _lib.NB_ERR_INVALID_ARG),
    (dict(L=0), _lib.NB_ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.NB_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.NB_ERR_INVALID_ARG),
    (dict(D=96), _lib.NB_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.NB_ERR_UNSUPPORTED),
    (dict(drop=0.1), _lib.NB_ERR_UNSUPPORTED),
])
def test_fwd_preflight(kw, status):
    assert _fwd(**kw) == status


def _bwd(owner_off, n_owner, att=FAKE, ws_bytes=1 << 20, **kw):
    a = dict(B=1, Hq=2, Hkv=1, L=8, S=16, D=64)
    a.update(kw)
    off = None if owner_off is None else (ctypes.c_int32 * len(owner_off))(*owner_off)
    return _lib.load().nb_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, a["B"], a["Hq"], a["Hkv"],
                                   a["L"], a["S"], a["D"], 0.125, -1, _lib.NB_BF16, FAKE, FAKE, FAKE,
                                   None if off is None else ctypes.cast(off, ctypes.c_void_p), n_owner, att,
                                   FAKE, ws_bytes, None)


def test_bwd_preflight():
    E = _lib.NB_ERR_INVALID_ARG
    assert _bwd([0, 16], 1, ws_bytes=8) == _lib.NB_ERR_WORKSPACE
    assert _bwd([0, 8, 15], 2) == E           # does not end at S
    assert _bwd([1, 8, 16], 2) == E           # does not start at 0
    assert _bwd([0, 9, 8, 16], 3) == E        # not ascending
    assert _bwd([0, 16], 1, att=None) == E    # no flag output
    assert _bwd(None, 65) == E                # too many owners
    assert _bwd([0, 16], 1, D=80) == _lib.NB_ERR_UNSUPPORTED


def test_segment_build_preflight():
    lib = _lib.load()
    need = lib.nb_segment_buffer_elems(1, 8, 16)
    assert lib.nb_segment_build(FAKE, None, 1, 16, 8, -1, FAKE, FAKE, need - 1, None) == _lib.NB_ERR_WORKSPACE
    assert lib.nb_segment_build(None, None, 1, 16, 8, -1, FAKE, FAKE, need, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_segment_build(FAKE, None, 1, 16, 20, -1, FAKE, FAKE, need, None) == _lib.NB_ERR_INVALID_ARG


def test_workload_generators_deterministic_and_shaped():
    for c in range(1, 6):
        w = wl.get(c)
        a, b = wl.make_doc_map(w), wl.make_doc_map(w)
        assert np.array_equal(a.doc_ids, b.doc_ids)
        assert a.doc_ids.shape == (w.B, a.S) and a.doc_ids.dtype == np.int32
        assert a.owner_off[0] == 0 and a.owner_off[-1] == a.S
        if w.mode != "halo":
            assert a.S == w.q_start + w.L
        else:
            assert w.L <= a.S <= 2 * w.L
        if w.pad_tail:
            assert a.pad_mask[:, -w.pad_tail:].all() and not a.pad_mask[:, :a.S - w.pad_tail].any()
    w = wl.get(1)
    q1 = wl.make_tensors(w, 256)
    q2 = wl.make_tensors(w, 256)
    assert all((x == y).all() for x, y in zip(q1, q2))
    assert q1[0].shape == (1, 2, 128, 64) and q1[1].shape == (1, 1, 256, 64)


def test_exchange_preflight_rejects_bad_arguments():
    """The exchange entry points check everything on the host first (no GPU needed:
    every call below returns before any launch)."""
    lib = _lib.load()
    assert lib.nb_exchange_plan_elems(0) == 0 and lib.nb_exchange_plan_elems(65) == 0
    P = 4
    n = lib.nb_exchange_plan_elems(P)
    assert n == 8 + 5 * P + 3 * P * P
    assert lib.nb_exchange_send_index_elems(P, 30) == 0          # N not a multiple of P
    assert lib.nb_exchange_send_index_elems(P, 32) == P * 32
    assert lib.nb_exchange_plan(None, None, 1, 32, P, FAKE, n, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_plan(FAKE, None, 1, 30, P, FAKE, n, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_plan(FAKE, None, 0, 32, P, FAKE, n, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_plan(FAKE, None, 1, 32, 65, FAKE, n, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_plan(FAKE, None, 1, 32, P, FAKE, n - 1, None) == _lib.NB_ERR_WORKSPACE
    assert lib.nb_exchange_send_index(FAKE, P, 32, FAKE, P * 32 - 1, None) == _lib.NB_ERR_WORKSPACE
    ptrs = (ctypes.c_void_p * P)(*([None] * P))
    # D * element size must be a multiple of 16 bytes; dtype must be known
    assert lib.nb_exchange_gather(FAKE, FAKE, 1, 1, 32, 4, P, _lib.NB_BF16, ptrs, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_gather(FAKE, FAKE, 1, 1, 32, 8, P, 7, ptrs, None) == _lib.NB_ERR_UNSUPPORTED
    assert lib.nb_exchange_scatter_add(ptrs, FAKE, 1, 1, 32, 8, P, _lib.NB_BF16, None, None) == \
        _lib.NB_ERR_INVALID_ARG
    bad = (ctypes.c_void_p * P)(*([FAKE + 4] + [None] * (P - 1)))   # misaligned rank buffer
    assert lib.nb_exchange_gather(FAKE, FAKE, 1, 1, 32, 8, P, _lib.NB_BF16, bad, None) == _lib.NB_ERR_INVALID_ARG
    assert lib.nb_exchange_gather(FAKE, FAKE, 300, 300, 32, 8, P, _lib.NB_BF16, ptrs, None) == \
        _lib.NB_ERR_INVALID_ARG                                      # B * C > 65535


def test_noalloc_backward_rejects_sizes_beyond_its_static_workspace():
    """nb_attn_bwd_noalloc: 8 MiB of static workspace; sizes whose workspace would
    exceed it are refused with NB_ERR_WORKSPACE before any HIP call (the pointers
    below are never dereferenced: the preflight returns first)."""
    lib = _lib.load()
    cap = lib.nb_attn_bwd_noalloc_max_workspace_bytes()
    assert cap == 8 << 20
    fake = ctypes.c_void_p(1 << 20)                      # non-null, 16-byte aligned, never used
    def call(B, Hq, Hkv, L, S, D):
        return lib.nb_attn_bwd_noalloc(fake, fake, fake, fake, fake, None, fake, fake, None, B, Hq, Hkv, L, S, D,
                                       D ** -0.5, -1, _lib.NB_BF16, fake, fake, fake, None, 0, None, None)
    # Delta alone: 64 heads x 40000 rows x 4 bytes > 8 MiB
    assert lib.nb_attn_bwd_workspace_bytes(1, 64, 8, 40000, 40000, 128, _lib.NB_BF16) > cap
    assert call(1, 64, 8, 40000, 40000, 128) == _lib.NB_ERR_WORKSPACE
    # the other checks come first, as for nb_attn_bwd
    assert call(1, 6, 4, 100, 200, 128) == _lib.NB_ERR_INVALID_ARG      # Hq % Hkv != 0
    assert call(1, 8, 2, 100, 200, 96) == _lib.NB_ERR_UNSUPPORTED       # head dim
    # the largest workload here fits (config 4: 32 heads x 8192 rows, 65536 keys)
    assert lib.nb_attn_bwd_workspace_bytes(1, 32, 8, 8192, 65536, 128, _lib.NB_BF16) <= cap


def test_head_dim_512_only_on_the_ring_chunk_calls():
    """The global layers' head dim (512) is taken by nb_ring_chunk_fwd / _bwd only; their
    backward's stored-dS workspace is then required (dQ = dS K is the only dQ pass at 512)."""
    lib = _lib.load()
    bf = _lib.NB_BF16
    assert _fwd(D=512) == _lib.NB_ERR_UNSUPPORTED
    assert _bwd([0, 16], 1, D=512) == _lib.NB_ERR_UNSUPPORTED
    ring = lib.nb_ring_chunk_bwd_workspace_bytes
    need = ring(1, 2, 1, 40, 64, 512, bf)
    assert need == lib.nb_attn_bwd_workspace_bytes(1, 2, 1, 40, 64, 512, bf) + _r256(2 * 64 * 160 * 2)
    def rbwd(ws_bytes, D=512):
        return lib.nb_ring_chunk_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 2, 1, 40, 64, D, 128, 64,
                                     D ** -0.5, bf, FAKE, FAKE, FAKE, 0, FAKE, ws_bytes, None)
    assert rbwd(need - 1) == _lib.NB_ERR_WORKSPACE          # refused before any launch
    assert rbwd(need, D=1024) == _lib.NB_ERR_UNSUPPORTED
    # a dS band over 2 GiB (32 heads x 8192 rows x 8288 keys x 2 bytes): unsupported at 512
    assert lib.nb_ring_chunk_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 32, 8, 8192, 8192, 512, 8192, 0,
                                 512 ** -0.5, bf, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == _lib.NB_ERR_UNSUPPORTED
