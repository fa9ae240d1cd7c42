#!/usr/bin/env python3
"""Throughput of one context-parallel rank's neighbourhood attention on one MI355X.

One step is the whole hot path over one batch of synthetic input: pad fold +
segment build, forward (O, LSE), backward (Delta and work orders, then the dQ
and dK/dV passes with the GQA reduction in one persistent grid) and the
per-owner attended flags -- all on the device, no host synchronisation inside
the step.  Inputs are resident in HBM before the
timed region starts.

Default workload: the Gemma-style sliding layer at rank 3 of a 4-way ring
(B=1, Hq=16, Hkv=8, D=256, L=4096, S=16384, window 1024, geometric doc lengths
with mean 2048), bf16.  The metric is useful fwd+bwd TFLOP/s with
useful FLOPs = 14 * D * Hq * pairs (4D forward + 10D backward per allowed
(query, key) pair per q head), pairs counted exactly from the seeded doc map.

Prints ONE JSON line.  Only the `cpu_baseline` leg touches the fp64 oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "fwd+bwd useful TFLOP/s per shard; % of bf16 MFMA peak (MI355X)"

# kernel -> (symbol substring in rocprof, source file, algorithmic FLOPs per allowed pair per q head / D)
KERNELS = {
    "attn_fwd": ("attn_fwd_kernel", "attn_fwd.hip", 4),     # S = QK^T, O = PV
    # one persistent grid for both backward passes: S, dP, dV = P^T dO, dK = dS^T Q, dQ = dS K
    # (the dQ pass's recompute of S and dP is not counted)
    "bwd_main": ("bwd_kernel", "attn_bwd.hip", 10),
}


RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # ~312: below it a step is HBM-bound
PEAK_FLOP_PER_CLK = 256 * 4096          # 256 CUs x 4096 dense bf16 FLOP per clock per CU


def stats(x) -> dict:
    """Median, min, p90 and mean of per-iteration times (ms)."""
    import numpy as np

    x = np.asarray(x, dtype=np.float64)
    return {"median": round(float(np.median(x)), 5), "min": round(float(x.min()), 5),
            "p90": round(float(np.percentile(x, 90)), 5), "mean": round(float(x.mean()), 5)}


def time_iters(stream, body, n_events, iters, scratch):
    """Per-iteration times (ms) of `body(events)` [iters, n_events]: each iteration gets its own events on the
    launch stream; with `scratch`, a write of the whole scratch buffer precedes every iteration (not timed)."""
    import numpy as np
    import torch

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events + 1)] for _ in range(iters)]
    torch.cuda.synchronize()
    for s in range(iters):
        if scratch is not None:
            scratch.fill_(s & 0x7F)
        body(evs[s])
    torch.cuda.synchronize()
    return np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(n_events)] for s in range(iters)])


def accounting(lib, segbuf, B, Hq, Hkv, L, S, D, W, dev) -> dict:
    """Exact allowed pairs per head and compulsory HBM bytes from the device segment buffer.

    Every real row's band is [max(row_klo, p - W), p]; a key is covered if some band holds it.  Compulsory bytes
    (bf16 tensors, fp32 LSE / Delta): forward reads Q and the covered K/V rows and writes O and LSE; the
    backward reads Q, dO, O, LSE and the covered K/V rows and writes dQ and every row of dK/dV (zeros included).
    Per kernel: the prep reads dO and O and writes Delta; bwd_main reads Q, dO, LSE, Delta and covered K/V and
    writes dQ, dK, dV."""
    import torch

    off_klo = lib.nb_segment_offset_row_klo(B, L)
    klo = segbuf[off_klo:off_klo + B * L].view(B, L).long()
    pos = (S - L + torch.arange(L, device=dev)).view(1, L).expand(B, L)
    lo = klo if W < 0 else torch.maximum(klo, pos - W)
    real = lo <= pos
    pairs = int(torch.clamp(pos - lo + 1, min=0).sum().item())
    # covered keys: difference array over the bands of the real rows
    diff = torch.zeros((B, S + 1), dtype=torch.int64, device=dev)
    ones = real.long()
    diff.scatter_add_(1, torch.where(real, lo, torch.full_like(lo, S)), ones)
    diff.scatter_add_(1, torch.where(real, pos + 1, torch.full_like(lo, S)), -ones)
    covered = int((torch.cumsum(diff, dim=1)[:, :S] > 0).sum().item())
    e = 2
    act = B * Hq * L * D * e          # one [B, Hq, L, D] tensor
    kv_cov = covered * Hkv * D * e    # covered rows of K (or V)
    kv_all = B * Hkv * S * D * e
    row32 = B * Hq * L * 4            # LSE or Delta
    by = {
        "attn_fwd": act + 2 * kv_cov + act + row32,
        "bwd_prep": 2 * act + row32,
        "bwd_main": 2 * act + 2 * row32 + 2 * kv_cov + act + 2 * kv_all,
        "owner_flags": 0,
    }
    step = (act + 2 * kv_cov + act + row32) + (3 * act + row32 + 2 * kv_cov + act + 2 * kv_all)
    by["step"] = step
    return {"pairs": pairs, "covered_keys": covered, "bytes": by, "ai": 14.0 * D * Hq * pairs / step}


def _sclk_path(index: int = 0):
    """sysfs DPM table of the GPU torch calls cuda:index (matched by PCI domain/bus/device), or None."""
    import glob

    import torch

    pr = torch.cuda.get_device_properties(index)
    want = (int(pr.pci_domain_id), int(pr.pci_bus_id), int(pr.pci_device_id))
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        addr = os.path.basename(os.path.realpath(os.path.dirname(path)))      # e.g. 0000:75:00.0
        m = re.match(r"([0-9a-fA-F]+):([0-9a-fA-F]+):([0-9a-fA-F]+)\.", addr)
        if m and tuple(int(x, 16) for x in m.groups()) == want:
            return path
    return None


def _read_sclk(path):
    """Current shader clock (MHz): the starred level of the DPM table."""
    try:
        with open(path) as fh:
            for line in fh:
                if "*" in line:
                    m = re.search(r"(\d+(?:\.\d+)?)\s*mhz", line, re.I)
                    return float(m.group(1)) if m else None
    except OSError:
        return None
    return None


def sample_sclk(body, stream, seconds: float = 1.5):
    """Median shader clock (MHz) read from the GPU's sysfs DPM table every few ms while `body` runs back to
    back for `seconds` (a thread reading a file: no child process); None where the table is not readable."""
    import threading

    import torch

    path = _sclk_path(torch.cuda.current_device())
    if path is None or _read_sclk(path) is None:
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            v = _read_sclk(path)
            if v is not None:
                samples.append(v)
            time.sleep(0.005)

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            body()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    if not samples:
        return None
    samples.sort()
    return samples[len(samples) // 2]


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_source_hash(fname: str) -> str:
    """First 16 hex digits of the sha256 over a kernel source and the local headers it includes (recursively,
    in include order): a profile taken from other code no longer matches."""
    csrc = os.path.join(ROOT, "sliding_window_attention_fold_amd", "csrc")
    h = hashlib.sha256()
    seen = []

    def visit(f):
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            return
        seen.append(f)
        with open(os.path.join(csrc, f), "rb") as fh:
            data = fh.read()
        h.update(data)
        for m in re.finditer(rb'^#include "([^"]+)"', data, re.M):
            visit(m.group(1).decode())

    visit(fname)
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, source: str = ""):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != kernel_source_hash(source or KERNELS[kernel][1]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, dm, tensors, rows: int, kv_heads: int):
    """The fp64 oracle (as it stands) on a bounded sample: the first `kv_heads` kv heads with their q heads,
    the first `rows` query rows, every key of the neighbourhood."""
    import numpy as np
    from oracle import nbattn_oracle as orc

    try:
        from threadpoolctl import threadpool_info

        cores = sum(int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    q, k, v, do = tensors
    nkv = max(1, min(kv_heads, w.Hkv))
    nq = nkv * w.g
    folded = orc.fold_pad(dm.doc_ids, dm.pad_mask)
    sel = np.arange(min(rows, w.L))
    t0 = time.perf_counter()
    orc.attention_forward(q[:, :nq], k[:, :nkv], v[:, :nkv], folded, w.window, w.D ** -0.5, rows=sel)
    orc.attention_backward(q[:, :nq], k[:, :nkv], v[:, :nkv], do[:, :nq], folded, w.window, w.D ** -0.5,
                           rows=sel)
    dt = time.perf_counter() - t0
    M = orc.allow_mask(folded, w.L, w.window, rows=sel)[:, 0] & orc.real_rows(folded, w.L)[:, sel][:, :, None]
    pairs = int(M.sum())
    flops = 14.0 * w.D * nq * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"fp64 numpy oracle fwd+bwd, kv heads [0,{nkv}) of {w.Hkv} ({nq} of {w.Hq} q heads), "
                      f"query rows [0,{len(sel)}) of {w.L}, all {dm.S} keys; {pairs} allowed pairs per head; "
                      f"{dt:.1f} s"}


def calibration_copy(mib: int, dev) -> None:
    """One plain copy of `mib` MiB read + `mib` MiB written, through the library's own 16-byte streaming copy
    (the exchange gather of a one-rank world whose single document covers everything), so that hardware byte
    counters can be scaled by what they read for the same access width."""
    import torch

    from sliding_window_attention_fold_amd import exchange as xg

    n = (mib << 20) // 256                      # tokens of 128 bf16
    plan = xg.exchange_plan(torch.ones((1, n), dtype=torch.int32, device=dev), 1)
    xg.needed_gather(torch.zeros((1, 1, n, 128), dtype=torch.bfloat16, device=dev), plan)
    torch.cuda.synchronize()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows of the oracle sample")
    ap.add_argument("--cpu-kv-heads", type=int, default=4, help="kv heads (with their q heads) of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain copy of this many MiB with the library's 16-byte streaming "
                         "copy (counter calibration)")
    ap.add_argument("--part", choices=["attention", "exchange", "ring"], default="attention",
                    help="attention: the hot path (default); exchange: the emulated needed-range K/V exchange; "
                         "ring: the global-layer ring (per-chunk attention, online merges)")
    ap.add_argument("--ring-config", type=int, default=2,
                    help="ring workload whose world the global-layer ring runs on (default 2)")
    ap.add_argument("--ring-head-dim", type=int, default=512,
                    help="head dim of the global-layer ring (default 512, the global layers'; 64/128/256 also run)")
    ap.add_argument("--kv", choices=["concat", "chunks"], default="concat",
                    help="concat: K/V as one neighbourhood buffer (default); chunks: the window-trimmed owner "
                         "chunks read in place (ring workloads)")
    ap.add_argument("--exchange-config", type=int, default=4,
                    help="workload whose world the exchange part emulates (default 4: 8 ranks, one document)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU "
              "path: each context-parallel rank's local attention is one GPU's work", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1)", file=sys.stderr)
        return 2

    if args.part == "exchange":
        return exchange_main(args)
    if args.part == "ring":
        return ring_main(args)
    if args.kv == "chunks":
        return chunks_main(args)

    import numpy as np
    import torch

    from sliding_window_attention_fold_amd import _lib
    from sliding_window_attention_fold_amd import workloads as wl

    lib = _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = wl.get(args.config)
    dm = wl.make_doc_map(w)
    q, k, v, do = wl.make_tensors(w, dm.S, "bf16")
    B, Hq, Hkv, L, S, D, W = w.B, w.Hq, w.Hkv, w.L, dm.S, w.D, w.window
    scale = D ** -0.5

    ids_d = torch.from_numpy(dm.doc_ids).to(dev)
    pad_d = None if dm.pad_mask is None else torch.from_numpy(dm.pad_mask).to(dev)
    qd, kd, vd, dod = (t.to(dev).contiguous() for t in (q, k, v, do))
    folded = torch.empty((B, S), dtype=torch.int32, device=dev)
    nseg = lib.nb_segment_buffer_elems(B, L, S)
    segbuf = torch.empty((nseg,), dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    resid = torch.empty(qd.shape, dtype=torch.int8, device=dev)   # the forward's residual codes
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq = torch.empty_like(qd)
    dk = torch.empty_like(kd)
    dv = torch.empty_like(vd)
    ws_bytes = lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S, D, _lib.NB_BF16, W)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    n_owner = len(dm.owner_off) - 1
    attended = torch.empty((n_owner,), dtype=torch.uint8, device=dev)
    off_c = (ctypes.c_int32 * len(dm.owner_off))(*dm.owner_off)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    bf = _lib.NB_BF16

    calls = {
        "segment_build": lambda: lib.nb_segment_build(P(ids_d), P(pad_d), B, S, L, W, P(folded), P(segbuf), nseg,
                                                      sp),
        "attn_fwd": lambda: lib.nb_attn_fwd(P(qd), P(kd), P(vd), P(out), P(resid), P(lse), P(segbuf), B, Hq, Hkv, L,
                                            S, D, scale, W, 0.0, bf, None, 0, sp),
        "bwd_prep": lambda: lib.nb_attn_bwd_prep(P(dod), P(out), P(resid), P(segbuf), B, Hq, Hkv, L, S, D, W, bf,
                                                 P(ws), ws_bytes, sp),
        "bwd_main": lambda: lib.nb_attn_bwd_main(P(dod), P(qd), P(kd), P(vd), P(lse), P(segbuf), B, Hq, Hkv, L, S,
                                                 D, scale, W, bf, P(dq), P(dk), P(dv), P(ws), ws_bytes, sp),
        "owner_flags": lambda: lib.nb_owner_attended(P(segbuf), P(folded), B, L, S, ctypes.cast(off_c,
                                                     ctypes.c_void_p), n_owner, P(attended), sp),
        # the product entry point: prep (Delta, work orders and, in extra workgroups, the owner flags) + main
        "attn_bwd": lambda: lib.nb_attn_bwd(P(dod), P(qd), P(kd), P(vd), P(out), P(resid), P(lse), P(segbuf),
                                            P(folded), B, Hq, Hkv, L, S, D, scale, W, bf, P(dq), P(dk), P(dv),
                                            ctypes.cast(off_c, ctypes.c_void_p), n_owner, P(attended), P(ws),
                                            ws_bytes, sp),
    }
    names = ["segment_build", "attn_fwd", "bwd_prep", "bwd_main", "owner_flags"]
    fb = names[1:]           # the backward as its separate launches (per-kernel times, the roofline)
    step_calls = ["attn_fwd", "attn_bwd"]   # one fwd+bwd step through the product entry points

    def run(seq, events=None):
        for i, n in enumerate(seq):
            if events is not None:
                events[i].record(stream)
            st = calls[n]()
            if st != 0:
                raise _lib.NbError(st, n)
        if events is not None:
            events[len(seq)].record(stream)

    # exact useful pairs and compulsory bytes from the device segment buffer (accounting, outside the timed region)
    run(names)
    torch.cuda.synchronize()
    acct = accounting(lib, segbuf, B, Hq, Hkv, L, S, D, W, dev)
    pairs = acct["pairs"]
    useful = 14.0 * D * Hq * pairs

    for _ in range(args.warmup):
        run(names)
        run(step_calls)
    torch.cuda.synchronize()

    # Segment build alone (once per step in training, outside fwd+bwd).
    seg_ms = time_iters(stream, lambda ev: run(["segment_build"], ev), 1, args.steps, None)[:, 0]
    # Primary: every fwd+bwd iteration starts after a 512 MiB scratch write, so L2 and the MALL hold none of
    # its inputs.  Each iteration is bracketed by its own events.
    scratch = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    flushed = time_iters(stream, lambda ev: run(step_calls, ev), len(step_calls), args.steps, scratch)
    # Warm: the same iterations back to back (inputs partly cached from the previous iteration).
    warm = time_iters(stream, lambda ev: run(step_calls, ev), len(step_calls), args.steps, None)
    # The backward's launches one by one, after the same flush: per-kernel times and the roofline.
    split = time_iters(stream, lambda ev: run(fb, ev), len(fb), args.steps, scratch)
    split_warm = time_iters(stream, lambda ev: run(fb, ev), len(fb), args.steps, None)
    # The K timed steps as one bracket (barrier + synchronise on both sides), back to back, segment build
    # included: the whole hot path.
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        run(["segment_build"] + step_calls)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    hot_path_ms = t_start.elapsed_time(t_end) / args.steps
    sclk = sample_sclk(lambda: run(step_calls), stream)
    del scratch

    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev)

    fb_f = flushed.sum(axis=1)
    fb_w = warm.sum(axis=1)
    ms_step = float(np.median(fb_f))
    tflops = useful / (ms_step * 1e-3) / 1e12
    per_mean = {n: float(split[:, i].mean()) for i, n in enumerate(fb)}
    dom = max(KERNELS, key=lambda n: per_mean[n])
    dom_ms = per_mean[dom]
    bound = "mfma" if acct["ai"] >= RIDGE_FLOP_PER_BYTE else "hbm"
    traffic = read_traffic(dom, f"config{args.config}")
    if bound == "mfma":
        dom_flops = KERNELS[dom][2] * D * Hq * pairs
        achieved, peak, unit = dom_flops / (dom_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        algo = {"algorithmic_flop_per_launch": dom_flops}
    else:
        dom_bytes = acct["bytes"][dom]
        achieved, peak, unit = dom_bytes / (dom_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        algo = {"algorithmic_bytes_per_launch": dom_bytes}
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"config{args.config}: {w.name}", "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "L": L, "S": S,
            "window": W, "doc_lengths": list(w.doc_len), "pad_tail": w.pad_tail, "seed": w.seed,
            "pairs_per_head": pairs, "useful_flop_per_step": useful,
        },
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "step": "fwd+bwd through the product entry points (nb_attn_fwd, nb_attn_bwd: prep with the owner flags, "
                "main), each iteration after a 512 MiB scratch write; value and ms_per_step from the median",
        "fwd_ms": stats(flushed[:, 0]),
        "bwd_ms": stats(flushed[:, 1]),
        "fwd_bwd_ms": stats(fb_f),
        "fwd_bwd_warm_ms": stats(fb_w),
        "warm_tflops": round(useful / (float(np.median(fb_w)) * 1e-3) / 1e12, 3),
        "segment_build_ms": stats(seg_ms),
        "hot_path_back_to_back_ms": round(hot_path_ms, 5),
        "hot_path_tflops": round(useful / (hot_path_ms * 1e-3) / 1e12, 3),
        "ms_per_kernel": {n: stats(split[:, i]) for i, n in enumerate(fb)},
        "ms_per_kernel_warm": {n: round(float(np.median(split_warm[:, i])), 5) for i, n in enumerate(fb)},
        "compulsory_bytes_per_step": acct["bytes"]["step"],
        "hbm_gbs_compulsory": round(acct["bytes"]["step"] / (ms_step * 1e-3) / 1e9, 1),
        "arithmetic_intensity": round(acct["ai"], 1),
        "sclk_mhz": sclk,
        "pct_of_bf16_peak_at_sclk": (None if not sclk else
                                     round(100.0 * tflops / (PEAK_FLOP_PER_CLK * sclk * 1e6 / 1e12), 2)),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "kernel": dom, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
            **algo,
            "avg_launch_ms": round(dom_ms, 5),
            "traffic_gbs": None if traffic is None else round(traffic / (dom_ms * 1e-3) / 1e9, 1),
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, dm, (q, k, v, do), args.cpu_rows, args.cpu_kv_heads)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def chunks_main(args) -> int:
    """The same workload with K/V read in place from the owner chunks, trimmed to the keys the left window
    reaches (no concatenated neighbourhood): one step = segment build over the trimmed neighbourhood,
    nb_attn_fwd_chunks, nb_attn_bwd_chunks (which also writes whole chunk-gradient buffers and the
    per-chunk attended flags).  Same useful FLOPs as the concatenated step."""
    import numpy as np
    import torch

    from sliding_window_attention_fold_amd import _lib
    from sliding_window_attention_fold_amd import api
    from sliding_window_attention_fold_amd import workloads as wl

    lib = _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = wl.get(args.config)
    if w.mode != "ring":
        print("--kv chunks needs a ring workload", file=sys.stderr)
        return 2
    dm = wl.make_doc_map(w)
    q, k, v, do = wl.make_tensors(w, dm.S, "bf16")
    B, Hq, Hkv, L, S, D, W = w.B, w.Hq, w.Hkv, w.L, dm.S, w.D, w.window
    scale = D ** -0.5
    C = len(dm.owner_off) - 1
    kd, vd = k.to(dev), v.to(dev)
    k_chunks = [kd[:, :, dm.owner_off[c]:dm.owner_off[c + 1]].contiguous() for c in range(C)]
    v_chunks = [vd[:, :, dm.owner_off[c]:dm.owner_off[c + 1]].contiguous() for c in range(C)]
    del kd, vd
    chunks = api.ring_window_chunks(k_chunks, v_chunks, W)
    n = len(chunks)
    S2 = sum(c.length for c in chunks)
    nb0 = S - S2
    ids_d = torch.from_numpy(np.ascontiguousarray(dm.doc_ids[:, nb0:])).to(dev)
    pad_d = None if dm.pad_mask is None else torch.from_numpy(np.ascontiguousarray(dm.pad_mask[:, nb0:])).to(dev)
    qd, dod = q.to(dev).contiguous(), do.to(dev).contiguous()
    folded = torch.empty((B, S2), dtype=torch.int32, device=dev)
    nseg = lib.nb_segment_buffer_elems(B, L, S2)
    segbuf = torch.empty((nseg,), dtype=torch.int32, device=dev)
    out, resid = torch.empty_like(qd), torch.empty(qd.shape, dtype=torch.int8, device=dev)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq = torch.empty_like(qd)
    dks = [torch.empty_like(c.k) for c in chunks]
    dvs = [torch.empty_like(c.v) for c in chunks]
    att = torch.empty((n,), dtype=torch.uint8, device=dev)
    ws_bytes = lib.nb_attn_bwd_workspace_bytes_window(B, Hq, Hkv, L, S2, D, _lib_bf16(), W)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    Pn, In = ctypes.c_void_p * n, ctypes.c_int32 * n
    kp, vp = Pn(*[c.k.data_ptr() for c in chunks]), Pn(*[c.v.data_ptr() for c in chunks])
    dkp, dvp = Pn(*[t.data_ptr() for t in dks]), Pn(*[t.data_ptr() for t in dvs])
    ln, st, rw = In(*[c.length for c in chunks]), In(*[c.start for c in chunks]), In(*[c.k.shape[2] for c in chunks])
    cv = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    Pp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    bf = _lib_bf16()
    calls = {
        "segment_build": lambda: lib.nb_segment_build(Pp(ids_d), Pp(pad_d), B, S2, L, W, Pp(folded), Pp(segbuf),
                                                      nseg, sp),
        "attn_fwd_chunks": lambda: lib.nb_attn_fwd_chunks(Pp(qd), cv(kp), cv(vp), cv(ln), cv(st), cv(rw), n,
                                                          Pp(out), Pp(resid), Pp(lse), Pp(segbuf), B, Hq, Hkv, L, S2,
                                                          D, scale, W, 0.0, bf, None, 0, sp),
        "attn_bwd_chunks": lambda: lib.nb_attn_bwd_chunks(Pp(dod), Pp(qd), cv(kp), cv(vp), cv(ln), cv(st), cv(rw), n,
                                                          Pp(out), Pp(resid), Pp(lse), Pp(segbuf), Pp(folded), B, Hq,
                                                          Hkv, L, S2, D, scale, W, bf, Pp(dq), cv(dkp), cv(dvp),
                                                          Pp(att), Pp(ws), ws_bytes, sp),
    }
    names = list(calls)

    def step(events=None):
        for i, nm in enumerate(names):
            if events is not None:
                events[i].record(stream)
            r = calls[nm]()
            if r != 0:
                raise _lib.NbError(r, nm)
        if events is not None:
            events[len(names)].record(stream)

    step()
    torch.cuda.synchronize()
    off_klo = lib.nb_segment_offset_row_klo(B, L)
    klo = segbuf[off_klo:off_klo + B * L].view(B, L).long()
    pos = (S2 - L + torch.arange(L, device=dev)).view(1, L)
    band_lo = klo if W < 0 else torch.maximum(klo, pos - W)
    pairs = int(torch.clamp(pos - band_lo + 1, min=0).sum().item())
    useful = 14.0 * D * Hq * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s_ in range(args.steps):
        step(evs[s_])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    per = {nm: float(np.mean([evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]))
           for i, nm in enumerate(names)}
    tflops = useful / (ms_step * 1e-3) / 1e12
    # For comparison only (outside the step): the copy the concatenated path needs first, K and V of every
    # causally valid chunk concatenated into one neighbourhood buffer (torch.cat, as the page's helper does).
    k_nb = torch.empty((B, Hkv, S, D), dtype=qd.dtype, device=dev)
    v_nb = torch.empty_like(k_nb)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cat(k_chunks, dim=2, out=k_nb)
    c0.record(stream)
    for _ in range(args.steps):
        torch.cat(k_chunks, dim=2, out=k_nb)
        torch.cat(v_chunks, dim=2, out=v_nb)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / args.steps
    rec = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "concat_copy_avoided_ms": round(copy_ms, 5),
        "config": {"workload": f"config{args.config}: {w.name}, K/V read in place from window-trimmed chunks",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "L": L, "S_concatenated": S, "S_trimmed": S2,
                   "chunks": [[c.start, c.length, int(c.k.shape[2])] for c in chunks], "window": W,
                   "pairs_per_head": pairs, "useful_flop_per_step": useful},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_call": {nm: round(per[nm], 5) for nm in names},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def ring_main(args) -> int:
    """The global-layer ring of one rank, every chunk resident on one GPU: the rank's queries against the K/V
    chunks of owners rank, rank-1, ..., 0 (own chunk causal, the rest non-causal, per-document masking, no
    window), each chunk's (out, lse) merged online (the cross chunks at their live rows), the merged output
    rounded, then every chunk's backward with the global out/lse (Delta formed once) summing dQ in fp32.
    Workload: --ring-config's world (default config 2: 4-way ring, rank 3, 4096-token chunks) as a full-attention
    layer.  Also timed, outside the step: the same attention as one pass over the chunk table."""
    import numpy as np
    import torch

    from sliding_window_attention_fold_amd import _lib
    from sliding_window_attention_fold_amd import workloads as wl

    lib = _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    import dataclasses

    w = dataclasses.replace(wl.get(args.ring_config), D=args.ring_head_dim)
    if w.mode != "ring":
        print("--part ring needs a ring workload", file=sys.stderr)
        return 2
    r, Lc = w.cp_rank, w.L
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    S = (r + 1) * Lc
    glob, pad = wl.global_doc_map(w)
    q, k, v, do = wl.make_tensors(w, S, "bf16")
    qd, dod = q.to(dev).contiguous(), do.to(dev).contiguous()
    order = [r] + list(range(r - 1, -1, -1))
    kc = [k[:, :, o * Lc:(o + 1) * Lc].contiguous().to(dev) for o in order]
    vc = [v[:, :, o * Lc:(o + 1) * Lc].contiguous().to(dev) for o in order]
    starts = [o * Lc for o in order]
    ids_d = torch.from_numpy(np.ascontiguousarray(glob[:, :S])).to(dev)
    pad_d = None if pad is None else torch.from_numpy(np.ascontiguousarray(pad[:, :S])).to(dev)
    bf = _lib.NB_BF16
    scale = D ** -0.5
    nseg = lib.nb_segment_buffer_elems(B, Lc, S)
    segbuf = torch.empty((nseg,), dtype=torch.int32, device=dev)
    folded = torch.empty((B, S), dtype=torch.int32, device=dev)
    out_step = torch.empty_like(qd)
    lse_step = torch.empty((B, Hq, Lc), dtype=torch.float32, device=dev)
    out_acc = torch.empty((B, Hq, Lc, D), dtype=torch.float32, device=dev)
    lse_acc = torch.empty((B, Hq, Lc), dtype=torch.float32, device=dev)
    out, resid = torch.empty_like(qd), torch.empty(qd.shape, dtype=torch.int8, device=dev)
    live_idx = torch.empty((B * Lc,), dtype=torch.int32, device=dev)
    n_live = torch.empty((1,), dtype=torch.int32, device=dev)
    dq_c = torch.empty_like(qd)
    dq_acc = torch.empty((B, Hq, Lc, D), dtype=torch.float32, device=dev)
    dks = [torch.empty_like(t) for t in kc]
    dvs = [torch.empty_like(t) for t in vc]
    # (D = 512 runs only the stored-dS backward, whose workspace holds the chunk-wide dS band)
    ws_bytes = (lib.nb_ring_chunk_bwd_workspace_bytes(B, Hq, Hkv, Lc, Lc, D, bf) if D >= 512
                else lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, Lc, Lc, D, bf))
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    Pp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    R = B * Hq * Lc
    q0 = r * Lc

    calls = [("segments", lambda: lib.nb_segment_build(Pp(ids_d), Pp(pad_d), B, S, Lc, -1, Pp(folded), Pp(segbuf),
                                                         nseg, sp)),
             ]
    for c, o in enumerate(order):
        calls.append((f"fwd_chunk{o}", lambda c=c: lib.nb_ring_chunk_fwd(
            Pp(qd), Pp(kc[c]), Pp(vc[c]), Pp(out_step), Pp(lse_step), Pp(segbuf), B, Hq, Hkv, Lc, Lc, D, q0,
            starts[c], scale, bf, sp)))
        if c == 0:
            calls.append((f"merge{o}", lambda: lib.nb_ring_merge(Pp(out_acc), Pp(lse_acc), Pp(out_step), Pp(lse_step),
                                                                 R, D, bf, 1, sp)))
        else:
            calls.append((f"live_rows{o}", lambda c=c: lib.nb_ring_live_rows(Pp(segbuf), B, Lc, Lc, q0, starts[c],
                                                                             Pp(live_idx), Pp(n_live), sp)))
            calls.append((f"merge_live{o}", lambda: lib.nb_ring_merge_live(
                Pp(out_acc), Pp(lse_acc), Pp(out_step), Pp(lse_step), Pp(live_idx), Pp(n_live), B * Lc, B, Hq, Lc,
                D, bf, sp)))
    calls.append(("finalize", lambda: lib.nb_ring_finalize(Pp(out_acc), Pp(out), Pp(resid), R, D, bf, sp)))
    for c, o in enumerate(order):
        # Delta once (first chunk); the chunks' dQ summed in fp32 by the kernels themselves
        fl = _lib.NB_RING_DQ_F32_SET if c == 0 else (_lib.NB_RING_DQ_F32_ADD | _lib.NB_RING_DELTA_READY)
        calls.append((f"bwd_chunk{o}", lambda c=c, fl=fl: lib.nb_ring_chunk_bwd(
            Pp(dod), Pp(qd), Pp(kc[c]), Pp(vc[c]), Pp(out), Pp(resid), Pp(lse_acc), Pp(segbuf), B, Hq, Hkv, Lc, Lc,
            D, q0, starts[c], scale, bf, Pp(dq_acc), Pp(dks[c]), Pp(dvs[c]), fl, Pp(ws), ws_bytes, sp)))

    def step(events=None):
        for i, (nm, fn) in enumerate(calls):
            if events is not None:
                events[i].record(stream)
            rc = fn()
            if rc != 0:
                raise _lib.NbError(rc, nm)
        if events is not None:
            events[len(calls)].record(stream)

    step()
    torch.cuda.synchronize()
    off_klo = lib.nb_segment_offset_row_klo(B, Lc)
    klo = segbuf[off_klo:off_klo + B * Lc].view(B, Lc).long()
    pos = (q0 + torch.arange(Lc, device=dev)).view(1, Lc)
    pairs = int(torch.clamp(pos - klo + 1, min=0).sum().item())
    useful = 14.0 * D * Hq * pairs
    bwd_flop = 10.0 * D * Hq * pairs
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s_ in range(args.steps):
        step(evs[s_])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    per = {nm: float(np.mean([evs[s_][i].elapsed_time(evs[s_][i + 1]) for s_ in range(args.steps)]))
           for i, (nm, _) in enumerate(calls)}
    bwd_ms = sum(v_ for nm, v_ in per.items() if nm.startswith("bwd_chunk"))
    tflops = useful / (ms_step * 1e-3) / 1e12

    # the same attention in one pass over the chunk table (outside the step, for comparison)
    asc = list(range(r + 1))
    Pn, In = ctypes.c_void_p * (r + 1), ctypes.c_int32 * (r + 1)
    kp = Pn(*[kc[order.index(o)].data_ptr() for o in asc])
    vp = Pn(*[vc[order.index(o)].data_ptr() for o in asc])
    dkp = Pn(*[dks[order.index(o)].data_ptr() for o in asc])
    dvp = Pn(*[dvs[order.index(o)].data_ptr() for o in asc])
    ln, st, rw = In(*([Lc] * (r + 1))), In(*([0] * (r + 1))), In(*([Lc] * (r + 1)))
    cv = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    lse1 = torch.empty((B, Hq, Lc), dtype=torch.float32, device=dev)
    ws1_bytes = lib.nb_attn_bwd_workspace_bytes(B, Hq, Hkv, Lc, S, D, bf) if D <= 256 else 1
    ws1 = torch.empty((ws1_bytes,), dtype=torch.uint8, device=dev)
    seg1 = torch.empty((lib.nb_segment_buffer_elems(B, Lc, S),), dtype=torch.int32, device=dev)
    fold1 = torch.empty((B, S), dtype=torch.int32, device=dev)

    def one_pass():
        for rc, nm in ((lib.nb_segment_build(Pp(ids_d), Pp(pad_d), B, S, Lc, -1, Pp(fold1), Pp(seg1), seg1.numel(),
                                             sp), "segments"),
                       (lib.nb_attn_fwd_chunks(Pp(qd), cv(kp), cv(vp), cv(ln), cv(st), cv(rw), r + 1, Pp(out),
                                               Pp(resid), Pp(lse1), Pp(seg1), B, Hq, Hkv, Lc, S, D, scale, -1, 0.0,
                                               bf, None, 0, sp), "fwd"),
                       (lib.nb_attn_bwd_chunks(Pp(dod), Pp(qd), cv(kp), cv(vp), cv(ln), cv(st), cv(rw), r + 1,
                                               Pp(out), Pp(resid), Pp(lse1), Pp(seg1), None, B, Hq, Hkv, Lc, S, D,
                                               scale, -1, bf, Pp(dq_c), cv(dkp), cv(dvp), None, Pp(ws1), ws1_bytes,
                                               sp), "bwd")):
            if rc != 0:
                raise _lib.NbError(rc, nm)

    one_ms = None
    if D <= 256:   # the chunk-table calls take head dims up to 256
        one_pass()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.steps):
            one_pass()
        c1.record(stream)
        torch.cuda.synchronize()
        one_ms = c0.elapsed_time(c1) / args.steps

    rec = {
        "metric": "global-layer ring fwd+bwd useful TFLOP/s per shard; % of bf16 MFMA peak (MI355X)",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"config{args.ring_config} world as a global (full-attention) layer: ring rank {r} of "
                               f"{w.cp_size}, {r + 1} chunks of {Lc} tokens, per-chunk attention + online merges",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "chunk": Lc, "chunks": r + 1, "window": -1,
                   "doc_lengths": list(w.doc_len), "pairs_per_head": pairs, "useful_flop_per_step": useful},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_call": {nm: round(v_, 5) for nm, v_ in per.items()},
        "one_pass_ms": None if one_ms is None else round(one_ms, 5),
        "roofline": {"kernel": "per-chunk backward (prep + main, all chunks)", "bound": "mfma",
                     "achieved": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_step": bwd_flop},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import ring_oracle as ro
        rows = min(Lc, args.cpu_rows)
        nh = min(Hq, 4)                     # q heads 0 .. nh-1 and their kv heads
        qs, dos = q[:, :nh, :rows], do[:, :nh, :rows]
        kv_h = max(1, nh // (Hq // Hkv))
        ids_f = glob[:, :S].copy()
        if pad is not None:
            ids_f[pad[:, :S] != 0] = 0
        q_ids = ids_f[:, q0:q0 + rows]
        t_start = time.perf_counter()
        acc = lacc = None
        for o in order:
            so, sl = ro.chunk_forward(qs, k[:, :kv_h, o * Lc:(o + 1) * Lc], v[:, :kv_h, o * Lc:(o + 1) * Lc], q_ids,
                                      ids_f[:, o * Lc:(o + 1) * Lc], q0, o * Lc, o == r, scale)
            acc, lacc = ro.merge(acc, lacc, so, sl)
        for o in order:
            ro.chunk_backward(qs, k[:, :kv_h, o * Lc:(o + 1) * Lc], v[:, :kv_h, o * Lc:(o + 1) * Lc], dos, acc, lacc,
                              q_ids, ids_f[:, o * Lc:(o + 1) * Lc], q0, o * Lc, o == r, scale)
        dt = time.perf_counter() - t_start
        m = ro.chunk_mask(q_ids, ids_f[:, :S], q0, 0, True)
        sample_pairs = int(m.sum()) * nh
        rec["cpu_baseline"] = {"value": round(14.0 * D * sample_pairs / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": torch.get_num_threads(), "kind": "oracle",
                               "sample": f"fp64 numpy ring oracle, q heads 0-{nh - 1}, query rows 0-{rows - 1} of the shard, "
                                         f"all {r + 1} chunks, forward + merges + backward; {dt:.1f} s"}
    print(json.dumps(rec), flush=True)
    return 0


def _lib_bf16() -> int:
    from sliding_window_attention_fold_amd import _lib
    return _lib.NB_BF16


def exchange_main(args) -> int:
    """The needed-range K/V exchange of one layer, emulated for every rank of the world on one GPU: plan
    and send index from the replicated doc ids, every rank's received K range (gather), and the backward
    index_add of every rank's dK range (scatter_add).  Workload: the single long document of the needed-range
    world (8 ranks of 8192 tokens, K [1, 8, 65536, 128] bf16), or --exchange-config's world.  HBM-bound; the roofline
    is the gather's algorithmic bytes (every received token read once and written once)."""
    import numpy as np
    import torch

    from sliding_window_attention_fold_amd import _lib
    from sliding_window_attention_fold_amd import exchange as xg
    from sliding_window_attention_fold_amd import workloads as wl

    lib = _lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = args.exchange_config
    w = wl.get(cfg)
    ids, pad = wl.global_doc_map(w)
    Bn, N = ids.shape
    P, C, D = w.cp_size, w.Hkv, w.D
    ids_d = torch.from_numpy(ids).to(dev)
    pad_d = None if pad is None else torch.from_numpy(pad).to(dev)
    plan = xg.exchange_plan(ids_d, P, pad_d)
    g = torch.Generator("cpu").manual_seed(w.seed)
    x = torch.randn((Bn, C, N, D), generator=g).to(torch.bfloat16).to(dev)
    recv = [torch.empty((Bn, C, int(R), D), dtype=x.dtype, device=dev) for R in plan.recv_len]
    grads = [torch.randn(t.shape, generator=g).to(torch.bfloat16).to(dev) for t in recv]
    gx = torch.empty_like(x)
    n_plan = lib.nb_exchange_plan_elems(P)
    n_si = lib.nb_exchange_send_index_elems(P, N)
    si = torch.empty((n_si,), dtype=torch.int32, device=dev)
    Pp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    rp = (ctypes.c_void_p * P)(*[t.data_ptr() if t.numel() else None for t in recv])
    gp = (ctypes.c_void_p * P)(*[t.data_ptr() if t.numel() else None for t in grads])
    calls = {
        "plan": lambda: lib.nb_exchange_plan(Pp(ids_d), Pp(pad_d), Bn, N, P, Pp(plan.buf), n_plan, sp),
        "send_index": lambda: lib.nb_exchange_send_index(Pp(plan.buf), P, N, Pp(si), n_si, sp),
        "gather": lambda: lib.nb_exchange_gather(Pp(x), Pp(plan.buf), Bn, C, N, D, P, _lib.NB_BF16, rp, sp),
        "scatter_add": lambda: lib.nb_exchange_scatter_add(gp, Pp(plan.buf), Bn, C, N, D, P, _lib.NB_BF16, Pp(gx),
                                                           sp),
    }
    names = list(calls)

    def step(events=None):
        for i, n in enumerate(names):
            if events is not None:
                events[i].record(stream)
            st = calls[n]()
            if st != 0:
                raise _lib.NbError(st, n)
        if events is not None:
            events[len(names)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s in range(args.steps):
        step(evs[s])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    per = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
           for i, n in enumerate(names)}
    if args.copy_mib > 0:
        calibration_copy(args.copy_mib, dev)
    T = int(plan.recv_len.sum())
    row = C * D * 2
    gather_bytes = 2 * Bn * T * row
    scatter_bytes = Bn * (T + N) * row
    moved = gather_bytes + scatter_bytes
    rec = {
        "metric": "emulated needed-range K/V exchange, HBM GB/s (gather + index_add backward)",
        "value": round(moved / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"config{cfg} world: {w.name}", "cp_size": P, "B": Bn, "C": C, "N": N, "D": D,
                   "use_halo": plan.use_halo, "halo_size": plan.halo_size, "received_tokens": T,
                   "bytes_per_step": moved},
        "ms_per_kernel": {n: round(per[n], 5) for n in names},
        "roofline": {
            "kernel": "gather", "bound": "hbm", "achieved": round(gather_bytes / (per["gather"] * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gather_bytes / (per["gather"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": read_traffic("exchange_gather", f"config{cfg}world", "exchange.hip"),
            "algorithmic_bytes_per_launch": gather_bytes,
        },
    }
    if not args.no_cpu_baseline:
        from oracle import exchange_oracle as ex
        op = ex.a2a_plan(ids, pad, P)
        xs = x[:, :1].float().cpu().numpy()          # one of the C channels
        gs = [t[:, :1].float().cpu().numpy() for t in grads]
        tc = time.perf_counter()
        ex.a2a_forward(xs, op)
        ex.a2a_backward(gs, op, xs.shape)
        dt = time.perf_counter() - tc
        rec["cpu_baseline"] = {"value": round(moved / C / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"fp64 numpy exchange oracle (plan excluded), channel 0 of {C}, all "
                                         f"{P} ranks; {dt:.1f} s"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
