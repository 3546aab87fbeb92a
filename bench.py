#!/usr/bin/env python3
"""POET-X layer forward+backward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3]

A step is one pass of the layer's hot path on one batch: CNP forward of G_R and
G_P, the layer forward, the layer backward (which ends with the CNP backward).
The permutation merge runs once per inner phase, before the timed region, and
is timed separately.  Inputs are seeded synthetic data resident in HBM before
timing starts.  Prints ONE JSON line.

Timing: about 0.3 s of untimed steps bring the GPU from idle to its steady clocks (see
settle()), then W untimed warm-up steps, then exactly K steps between two device
synchronizations.  Inside that timed region the dominant kernel's launches (the W'
product) carry a start and a stop event bound to their own dispatch (the library's
per-thread recorder, hipExtLaunchKernel, events without a system-scope fence), and
one event marks each step boundary: `roofline` and the per-step median/min/max come
from the timed steps themselves.  The same K steps then run once unrecorded (the
cost of the recording) and once with every launch recorded (`phases`, the per-kernel
table: a recorded dispatch waits a few us on its events, so that pass's step time is
longer, while the kernels' own durations match an unrecorded kernel trace).

Besides the head workload (default 3) the default run also measures the other
workloads of the build: 4 (fast, mem), 5 (mem) and 2 (CNP blocks/s); the head
workload is also run with NULL activation permutations and as the pages' own fast
variant (which keeps only B).  --only-head skips all of that (profiling runs).

Extra modes used to make the committed profile summaries:
    --copy-calibration   time a plain 1 GiB device copy (the HBM counter calibration)
    --no-cpu             skip the CPU-oracle baseline leg
    --summarize-trace DB [JSON]      markdown kernel table from a rocprofv3 --kernel-trace database
                                     (with the traced run's JSON line: dominant kernel trace vs events)
    --summarize-counters F W CF CW [JSON]  HBM traffic per kernel from four rocprofv3 --pmc databases
                                     (FETCH_SIZE, WRITE_SIZE; then the same two counters taken on
                                     --copy-calibration); with the run's JSON line, traffic / algorithmic
    --summarize-pmc DB [DB ...]      per-kernel averages of any counters in --pmc databases
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "POET-X layer fwd+bwd tokens/s (4096², b=256) + % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
DOMINANT = "gemm_nt"


# ------------------------------------------------------------------ work model ----
def algorithmic(wl, variant, n, perms=True, keep_x=True):
    """Per-step algorithmic flops and HBM bytes of each kernel label: the minimum each kernel
    must compute and move (its operands read once, its results written once)."""
    di, do, b = wl.d_in, wl.d_out, wl.b
    nr, np_ = di // b, do // b
    ae = 2 if wl.act == "bf16" else 4
    we = {"bf16": 2, "f32": 4, "i8": 1}[wl.w]
    mem = variant == "mem"
    ops = {}

    def add(name, flops, nbytes):
        f, y = ops.get(name, (0.0, 0.0))
        ops[name] = (f + flops, y + nbytes)

    g_bytes_r, g_bytes_p = nr * b * b * ae, np_ * b * b * ae
    fronts = 2 if mem else 1  # mem recomputes gather, R-side apply and the forward GEMM
    for _ in range(fronts):
        if perms:
            add("permute_cols", 0, 2 * n * di * ae)                               # gather X
        add("block_apply", 2.0 * n * di * b, 2 * n * di * ae + g_bytes_r)
        add("gemm_nt", 2.0 * n * di * do, n * di * ae + do * di * we + n * do * ae)
    if perms and not mem and not keep_x:
        add("permute_cols", 0, 2 * n * di * ae)                                   # gather X again
    add("block_apply", 2.0 * n * do * b, 2 * n * do * ae + g_bytes_p)            # Z~ = B G_P
    if perms:
        add("permute_cols", 0, 2 * n * do * ae)                                   # scatter Z
        add("permute_cols", 0, 2 * n * do * ae)                                   # gather dZ
    add("block_apply_t", 2.0 * n * do * b, 2 * n * do * ae + g_bytes_p)          # dB
    add("block_grad", 2.0 * n * do * b, 2 * n * do * ae)                          # dG_P
    add("gemm_nn", 2.0 * n * di * do, n * do * ae + do * di * we + n * di * ae)   # dA
    add("block_apply_t", 2.0 * n * di * b, 2 * n * di * ae + g_bytes_r)          # dX~
    if perms:
        add("permute_cols", 0, 2 * n * di * ae)                                   # scatter dX
    add("block_grad", 2.0 * n * di * b, 2 * n * di * ae)                          # dG_R
    # CNP, both sides (nb blocks), at the method's own product count (forward 2 b^3-products
    # by Horner, backward 6; 2 b^3 flops each) and its minimum bytes: theta in and G out
    # (forward), theta and dG in and dtheta out (backward).
    nb = nr + np_
    p, bb = b * (b - 1) // 2, b * b
    add("cnp_fwd", 4.0 * b ** 3 * nb, nb * 4 * p + nb * ae * bb)
    add("cnp_bwd", 12.0 * b ** 3 * nb, nb * 4 * (bb + 2 * p))
    return ops


# kernel labels of the library -> the algorithmic group they carry
LABEL_GROUP = {"unpack_skew": "cnp_fwd", "cnp_fwd_chain": "cnp_fwd", "cnp_fwd_mm": "cnp_fwd",
               "cnp_bwd5": "cnp_bwd",
               "cnp_bwd_mm": "cnp_bwd", "pack_skew_grad": "cnp_bwd", "reduce_parts": "block_grad",
               "gemm_tail_reduce": None, "transpose": None}


def survey_floor_ms(wl, variant, n):
    """The step's roofline floor with the activation permutations fused into the block
    products: sum over the method's steps of max(flops / 2.5 PF/s, bytes / 8 TB/s), every
    product counted once in bf16, the CNP at its method flops (Horner 2 + 6 products)."""
    di, do, b = wl.d_in, wl.d_out, wl.b
    ae = 2 if wl.act == "bf16" else 4
    we = {"bf16": 2, "f32": 4, "i8": 1}[wl.w]
    nr, np_ = di // b, do // b
    nb, p, bb = nr + np_, b * (b - 1) // 2, b * b
    gr, gp = nr * bb * ae, np_ * bb * ae
    gemm = (2.0 * n * di * do, n * di * ae + di * do * we + n * do * ae)
    phases = [
        (4.0 * b ** 3 * nb, nb * 4 * p + nb * ae * bb),                      # S1 CNP forward
        (2.0 * n * di * b, 2 * n * di * ae + gr),                            # S2+S3 gather + apply R
        gemm,                                                                # S4
        (2.0 * n * do * b, 2 * n * do * ae + gp),                            # S5 apply P + scatter
        (4.0 * n * do * b, 3 * n * do * ae + gp + np_ * bb * 4),             # S7 P side
        gemm,                                                                # S8
        (4.0 * n * di * b, 3 * n * di * ae + gr + nr * bb * 4),              # S9 R side
        (12.0 * b ** 3 * nb, nb * 4 * (bb + 2 * p)),                         # S10 CNP backward
    ]
    if variant == "mem":
        phases += [(2.0 * n * di * b, 2 * n * di * ae + gr), gemm]          # S6 recompute
    t = sum(max(f / (PEAK_BF16_TFLOPS * 1e12), y / (PEAK_HBM_GBS * 1e9)) for f, y in phases)
    return t * 1e3


def unfused_floor_ms(wl, variant, n, perms=True, keep_x=True):
    """The same floor for the kernels as built: each permutation a separate pass over its
    activation (bytes per label from algorithmic())."""
    t = 0.0
    for f, y in algorithmic(wl, variant, n, perms, keep_x).values():
        t += max(f / (PEAK_BF16_TFLOPS * 1e12), y / (PEAK_HBM_GBS * 1e9))
    return t * 1e3


def step_flops(wl, variant, n):
    return sum(f for f, _ in algorithmic(wl, variant, n).values())


# ------------------------------------------------------------------ timing ----
def _sync():
    import torch
    torch.cuda.synchronize()


SETTLE_S = 0.3


def settle(st, seconds=None):
    """Untimed steps for `seconds` of wall time, ahead of the warm-up steps: an idle GPU
    comes back at low clocks and takes tens of ms of load to reach its steady ones (a
    kernel trace of the first steps after idle shows every kernel 5-8% slower)."""
    seconds = SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            st.step()
        _sync()


def time_steps(st, steps, warmup, record, only=None):
    """K steps between two synchronizations, an event at each step boundary; with
    `record`, the launches labelled `only` (every launch when None) carry dispatch-bound
    start/stop events."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    for _ in range(warmup):
        st.step()
    _sync()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if record:
        B.prof_read()  # clear
        B.prof_only(only)
        B.prof_enable(True)
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        st.step()
    ev[steps].record()
    _sync()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    rec = None
    if record:
        B.prof_enable(False)
        B.prof_only(None)
        rec = B.prof_read()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return wall, per, rec


def phase_table(rec, alg, steps):
    out = {}
    for name, (cnt, tot, mn, mx) in sorted(rec.items()):
        e = {"launches_per_step": cnt / steps, "avg_ms": tot / cnt, "min_ms": mn, "max_ms": mx,
             "ms_per_step": tot / steps}
        grp = LABEL_GROUP.get(name, name)
        if grp in alg and grp == name:
            f, y = alg[name]
            per = cnt / steps
            e["tflops"] = f / per / (e["avg_ms"] * 1e-3) / 1e12
            e["gbs"] = y / per / (e["avg_ms"] * 1e-3) / 1e9
            e["frac_mfma"] = e["tflops"] / PEAK_BF16_TFLOPS
            e["frac_hbm"] = e["gbs"] / PEAK_HBM_GBS
        out[name] = e
    # CNP groups: several launches carry one method step
    for grp in ("cnp_fwd", "cnp_bwd"):
        ms = sum(e["ms_per_step"] for k, e in out.items() if LABEL_GROUP.get(k) == grp)
        if ms > 0 and grp in alg:
            f, y = alg[grp]
            out[grp + " (all launches)"] = {
                "ms_per_step": ms, "tflops": f / (ms * 1e-3) / 1e12, "gbs": y / (ms * 1e-3) / 1e9,
                "frac_mfma": f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "frac_hbm": y / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return out


def flush_cache(buf):
    """Write 1 GiB: evicts the 256 MB Infinity Cache and the L2s."""
    buf.fill_(1)


def run_variant(wl, inputs, variant, steps, warmup, *, keep_wt, keep_x=True, perms=True, cold_steps=0):
    import torch
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.step import LayerStep
    st = LayerStep(wl, inputs, variant, transposed_weight=keep_wt, keep_x=keep_x, perms=perms)
    n = wl.n_tokens
    # the timed steps: only the dominant kernel's launches carry events (a recorded dispatch
    # waits a few us on its events' bookkeeping), then the same steps unrecorded, then once
    # more with every launch recorded for the per-kernel table
    settle(st)
    wall, per, rec_dom = time_steps(st, steps, warmup, record=True, only=DOMINANT)
    wall_off, per_off, _ = time_steps(st, steps, 1, record=False)
    wall_all, _, rec = time_steps(st, steps, 1, record=True)
    alg = algorithmic(wl, variant, n, perms, keep_x and st.saved_x is not None)
    floor_fused = survey_floor_ms(wl, variant, n)
    floor_unfused = unfused_floor_ms(wl, variant, n, perms, keep_x and st.saved_x is not None)
    v = {"ms_per_step": wall, "tokens_per_s": n / (wall * 1e-3),
         "step_ms": {"median": statistics.median(per), "min": min(per), "max": max(per),
                     "mean": sum(per) / len(per)},
         "ms_per_step_unrecorded": wall_off,
         "step_ms_unrecorded": {"median": statistics.median(per_off), "min": min(per_off),
                                "max": max(per_off)},
         "ms_per_step_all_recorded": wall_all,
         "w_merged_t": keep_wt, "kept_x": st.saved_x is not None, "activation_permutations": perms,
         "floor_fused_ms": floor_fused, "frac_of_fused_floor": floor_fused / wall,
         "floor_unfused_ms": floor_unfused, "frac_of_unfused_floor": floor_unfused / wall}
    phases = phase_table(rec, alg, steps)
    if rec_dom and DOMINANT in rec_dom:
        # the dominant kernel as timed inside the timed steps themselves
        phases[DOMINANT + " (timed steps)"] = phase_table({DOMINANT: rec_dom[DOMINANT]}, alg, steps)[DOMINANT]
    cold = None
    if cold_steps:
        # per-phase HBM figures with nothing left in the caches from the previous step
        fl = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        B.prof_read()
        acc = {}
        for _ in range(cold_steps):
            flush_cache(fl)
            _sync()
            B.prof_enable(True)
            st.step()
            _sync()
            B.prof_enable(False)
            for k, (c, t, mn, mx) in B.prof_read().items():
                a = acc.setdefault(k, [0, 0.0, mn, mx])
                a[0] += c; a[1] += t; a[2] = min(a[2], mn); a[3] = max(a[3], mx)
        cold = phase_table({k: tuple(a) for k, a in acc.items()}, alg, cold_steps)
        del fl
    del st
    torch.cuda.empty_cache()
    return v, phases, cold


def merge_time_ms(wl, inputs, reps=10, with_t=False):
    import torch
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.step import upload
    w = upload(inputs["w"] if wl.w != "i8" else inputs["w_q"], wl.w if wl.w != "i8" else "i8")
    s = upload(inputs.get("w_s"), "f32") if wl.w == "i8" else None
    pin, pout = upload(inputs["perm_in"], "i32"), upload(inputs["perm_out"], "i32")
    out = torch.empty_like(w)
    so = torch.empty_like(s) if s is not None else None
    ot = torch.empty((wl.d_in, wl.d_out), dtype=w.dtype, device=w.device) if with_t else None
    B.poetx_merge_perm(w, pout, pin, s, out, so, ot)
    _sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.poetx_merge_perm(w, pout, pin, s, out, so, ot)
    e1.record()
    _sync()
    ms = e0.elapsed_time(e1) / reps
    nbytes = (4 if with_t else 2) * w.numel() * w.element_size()
    return ms, nbytes / (ms * 1e-3) / 1e9


def fold_time_ms(wl, inputs, reps=10):
    """Phase-end fold (poetx_fold) at the workload's weight shape; None for int8."""
    if wl.w == "i8":
        return None
    import torch
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd.step import LayerStep
    st = LayerStep(wl, dict(inputs, x=inputs["x"][:64], dz=inputs["dz"][:64]), "mem")
    st.cnp()
    w_out = torch.empty_like(st.w_merged)
    B.poetx_fold(st.layer, w_out)
    _sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.poetx_fold(st.layer, w_out)
    e1.record()
    _sync()
    return e0.elapsed_time(e1) / reps


def adam_time_ms(wl, reps=20):
    """poetx_adam_step over the layer's packed theta (both sides), float32 state."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    n = (wl.d_in // wl.b + wl.d_out // wl.b) * (wl.b * (wl.b - 1) // 2)
    th = torch.zeros(n, device="cuda")
    g, m, v = torch.randn(n, device="cuda"), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    B.poetx_adam_step(th, g, m, v, lr=1e-3, step=1)
    _sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(reps):
        B.poetx_adam_step(th, g, m, v, lr=1e-3, step=t + 2)
    e1.record()
    _sync()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": ms, "params": n, "GB_s": 7 * 4 * n / (ms * 1e-3) / 1e9}


def measured_peaks(wl):
    """What this GPU sustains on a plain 1 GiB device copy and on the vendor library's
    GEMM (torch.matmul, hipBLASLt) at the W' product's shape."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    _sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    _sync()
    copy_gbs = 2 * n / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del a, b
    m, k, nn = wl.n_tokens, wl.d_in, wl.d_out
    x = torch.randn(m, k, device="cuda").to(torch.bfloat16)
    w = torch.randn(nn, k, device="cuda").to(torch.bfloat16)
    wt = w.t()
    y = torch.empty(m, nn, dtype=torch.bfloat16, device="cuda")
    for _ in range(10):
        torch.matmul(x, wt, out=y)
    _sync()
    ms = None
    for _ in range(5):  # the best of five batches of 20 (the library's clocks settle)
        e0.record()
        for _ in range(20):
            torch.matmul(x, wt, out=y)
        e1.record()
        _sync()
        t = e0.elapsed_time(e1) / 20
        ms = t if ms is None else min(ms, t)
    del x, w, wt, y
    torch.cuda.empty_cache()
    return {"copy_GB_s": copy_gbs, "library_gemm_TF_s": 2.0 * m * k * nn / (ms * 1e-3) / 1e12,
            "library_gemm_ms": ms, "library_gemm_shape": [m, nn, k],
            "how": "torch copy_ of 1 GiB (read + write bytes / time); torch.matmul bf16 (hipBLASLt) "
                   "X[N][d_in] @ W^T[d_in][d_out], best of 5 batches of 20 launches"}


def cpu_baseline(wl, inputs, target_s=15.0):
    """The fp64 oracle on host cores on a bounded token sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import poetx_oracle as O
    from orthogonal_reparameterized_amd import workloads as WL
    if wl.w == "i8":  # the oracle's W' is the merged int8 weight times its merged row scales
        qm, sm = O.merge_perm_int8(inputs["w_q"], inputs["w_s"], inputs["perm_out"], inputs["perm_in"])
        wm = O.dequantize_rows(qm, sm)
    else:
        wm = O.merge_perm(WL.to_f64(inputs["w"], wl.w), inputs["perm_out"], inputs["perm_in"])
    tr, tp = inputs["theta_r"].astype(np.float64), inputs["theta_p"].astype(np.float64)

    def run(n):
        x = WL.to_f64(inputs["x"][:n], wl.act)
        dz = WL.to_f64(inputs["dz"][:n], wl.act)
        t0 = time.perf_counter()
        O.poetx_step(x, dz, wm, tr, tp, wl.b, inputs["perm_in"], inputs["perm_out"])
        return time.perf_counter() - t0

    n = min(256, wl.n_tokens)
    t = run(n)
    while t < target_s / 4 and n < wl.n_tokens:
        n = min(wl.n_tokens, n * 4)
        t = run(n)
    reps = 1
    while t < 1.0:  # a workload that takes the oracle well under a second: repeat whole steps
        reps *= 2
        t = sum(run(n) for _ in range(reps))
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    what = (f"first {n} of {wl.n_tokens} tokens of the workload" if n < wl.n_tokens
            else f"all {n} tokens of the workload")
    steps = "one full oracle step" if reps == 1 else f"{reps} full oracle steps"
    return {"value": reps * n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, {steps} (CNP fwd, layer fwd, layer bwd, CNP bwd) in float64 NumPy, {t:.1f} s"}


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    _sync()
    for _ in range(3):
        b.copy_(a)
    _sync()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    _sync()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GB_s_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))


# ------------------------------------------------------------ profile summaries ----
KERNEL_SYMBOL_CANDIDATES = {  # kernel label -> substrings of the symbols that may carry it
    "gemm_nt": ("k_gemm4<", "k_gemm2<0,"),
}
KERNEL_SYMBOL = {  # kernel label -> substring of its symbol in traces (workload 3 shapes)
    "gemm_nt": "k_gemm2<0,", "gemm_nn": "k_gemm_pp<1,", "block_apply": "k_block_reg<256,32,7,false,8>",
    "block_apply_t": "k_block_reg<256,32,7,true,8>", "block_grad": "k_block_grad_stream<256,4,64,2>",
}
# the dominant kernel's sources: recorded counters stay valid while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "orthogonal_reparameterized_amd", "csrc", f)
                  for f in ("k_gemm2.hip", "lds_tiles.h")]


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload_key):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_workload{workload_key}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _short(name):
    return name.replace("(poetx::KArgs)", "").replace("poetx::", "").replace("void ", "")[:95]


def summarize_trace(db, bench_json=None):
    """Markdown kernel table of a --kernel-trace database; with the JSON line that the
    traced bench.py run printed, also the dominant kernel's trace average next to the
    recorder's average from the same timed steps."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                       "sum(duration) from kernels group by name order by sum(duration) desc").fetchall()
    tot = sum(r[5] for r in rows)
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, n, avg, mn, mx, sm in rows:
        print(f"| `{_short(name)}` | {n} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | {100 * sm / tot:.1f}% |")
    # a symbol that runs several shapes (the 256 x 256 kernel: W' products, batched block
    # products at b = 512) gets its launches split by grid (workgroups x batch)
    shapes = con.execute("select name, grid_x / workgroup_x, grid_z, count(*), avg(duration), min(duration), "
                         "max(duration) from kernels group by name, grid_x / workgroup_x, grid_z "
                         "order by name, grid_z, grid_x / workgroup_x").fetchall()
    multi = {r[0] for r in shapes if sum(1 for q in shapes if q[0] == r[0]) > 1}
    if multi:
        print()
        print("| kernel | workgroups x batch | launches | avg us | min us | max us |")
        print("|---|---|---:|---:|---:|---:|")
        for name, gx, gz, n, avg, mn, mx in shapes:
            if name in multi:
                print(f"| `{_short(name)}` | {gx} x {gz} | {n} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} |")
    if not bench_json:
        return
    line = [ln for ln in open(bench_json) if ln.startswith("{")][-1]
    d = json.loads(line)
    if "phases" not in d:  # the CNP microbenchmark
        print()
        print(f"bench.py in this run: forward {d['fwd_ms']:.3f} ms, backward {d['bwd_ms']:.3f} ms per call "
              f"over {d['config']['nblocks']} blocks of b = {d['config']['b']}: "
              f"{d['value'] / 1e3:.0f} K blocks/s.")
        return
    roof = d["roofline"]
    names = [r[0].replace(" ", "") for r in rows]
    sym = next(sm for sm in KERNEL_SYMBOL_CANDIDATES[roof["kernel"]] if any(sm in nm for nm in names))
    # unbatched launches only (batched ones of the same symbol are block products)
    durs = [r[1] for r in con.execute("select name, duration from kernels where grid_z = 1 order by start")
            if sym in r[0].replace(" ", "")]
    # the traced run (--only-head, one variant): settle steps, W warm-up steps, K timed steps
    # (this kernel recorded), 1 + K unrecorded, 1 + K all recorded, then 5 cold-cache steps;
    # the windows are counted back from the end
    k, w = d["steps"], d["warmup"]
    c = int(round(d["phases"][d["config"]["variant"]]["gemm_nt"]["launches_per_step"]))
    if d["variants"][d["config"]["variant"]].get("w_merged_t"):
        c *= 2  # the backward product runs the same kernel on W'^T
    end = len(durs) - 5 * c
    allrec = durs[end - k * c:end]
    unrec = durs[end - (2 * k + 1) * c:end - (k + 1) * c]
    timed = durs[end - (3 * k + 2) * c:end - (2 * k + 2) * c]

    def avg(v):
        return sum(v) / len(v) / 1e3 if v else float("nan")
    print()
    print(f"Dominant kernel `{roof['kernel']}` (`{sym}`, {c} launch(es) per step): trace average over the "
          f"timed steps' launches {avg(timed):.1f} us, over the unrecorded steps' {avg(unrec):.1f} us, over "
          f"the all-recorded steps' {avg(allrec):.1f} us; bench.py's event-timed average over its "
          f"{roof['launches']} launches in the timed steps {roof['avg_launch_ms'] * 1e3:.1f} us -> "
          f"{roof['achieved']:.0f} TFLOP/s, frac {roof['frac']:.3f}.  Step {d['ms_per_step']:.4f} ms "
          f"(median {d['step_ms']['median']:.4f}), {d['value'] / 1e6:.3f} M tokens/s; unrecorded "
          f"{d['variants'][d['config']['variant']]['ms_per_step_unrecorded']:.4f} ms.")


def _pmc_rows(db, counter=None):
    import sqlite3
    con = sqlite3.connect(db)
    q = "select kernel_name, counter_name, count(*), avg(value) from counters_collection"
    if counter:
        return con.execute(q + " where counter_name = ? group by kernel_name, counter_name", (counter,)).fetchall()
    return con.execute(q + " group by kernel_name, counter_name").fetchall()


def summarize_counters(fetch_db, write_db, copy_fetch_db, copy_write_db, bench_json=None):
    """HBM bytes per dispatch of every kernel in the run, scaled by what the same counters
    read on a 1 GiB copy; with the run's JSON line, next to the algorithmic bytes."""
    def pick(rows, match):
        for name, _, n, v in rows:
            if match in name.replace(" ", ""):
                return n, v
        raise SystemExit(f"no kernel matching {match}")

    copy_kib = float(1 << 30) / 1024
    _, cf = pick(_pmc_rows(copy_fetch_db, "FETCH_SIZE"), "copyBuffer")
    _, cw = pick(_pmc_rows(copy_write_db, "WRITE_SIZE"), "copyBuffer")
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    fetch = {r[0]: (r[2], r[3]) for r in _pmc_rows(fetch_db, "FETCH_SIZE")}
    write = {r[0]: (r[2], r[3]) for r in _pmc_rows(write_db, "WRITE_SIZE")}
    print(f"copy_fetch_kib_raw = {cf:.1f}  (1 GiB copy reads {copy_kib:.0f} KiB)")
    print(f"copy_write_kib_raw = {cw:.1f}  (1 GiB copy writes {copy_kib:.0f} KiB)")
    print(f"fetch_scale = {f_scale:.4f}")
    print(f"write_scale = {w_scale:.4f}")
    print()
    print("| kernel | dispatches | fetch MB | write MB | traffic MB per dispatch |")
    print("|---|---:|---:|---:|---:|")
    for name in sorted(fetch, key=lambda k: -fetch[k][1]):
        nf, f = fetch[name]
        _, w = write.get(name, (0, 0.0))
        tr = (f * f_scale + w * w_scale) * 1024
        print(f"| `{_short(name)}` | {nf} | {f * f_scale * 1024 / 1e6:.1f} | {w * w_scale * 1024 / 1e6:.1f} | "
              f"{tr / 1e6:.1f} |")
    sym = KERNEL_SYMBOL[DOMINANT]
    _, f = pick(_pmc_rows(fetch_db, "FETCH_SIZE"), sym)
    _, w = pick(_pmc_rows(write_db, "WRITE_SIZE"), sym)
    print()
    print(f"kernel_label = {DOMINANT}")
    print(f"kernel_symbol_match = {sym}")
    print(f"traffic_bytes_per_launch = {(f * f_scale + w * w_scale) * 1024:.0f}")
    print(f"kernel_sources = {' + '.join(os.path.relpath(f, ROOT) for f in KERNEL_SOURCES)}")
    print(f"kernel_source_sha = {kernel_source_sha()}")


def summarize_pmc(*dbs):
    """Per-kernel averages of the counters in --pmc databases; where a kernel has
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE, its MFMA-busy fraction (busy cycles summed
    over the SIMDs / (GPU-active cycles per XCD x SIMDs)), and with SQ_INSTS_VALU_MFMA_MOPS_BF16 its
    bf16 MFMA flops per dispatch (MOPS x 512)."""
    import torch
    simds = 4 * (torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256)
    per = {}
    print("| kernel | counter | dispatches | average per dispatch |")
    print("|---|---|---:|---:|")
    for db in dbs:
        for name, ctr, n, v in sorted(_pmc_rows(db), key=lambda r: (r[0], r[1])):
            print(f"| `{_short(name)}` | {ctr} | {n} | {v:.4g} |")
            per.setdefault(name, {})[ctr] = v
    rows = [(k, d) for k, d in per.items() if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d]
    if rows:
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (about 8 x the kernel's shader clocks)
        print()
        print(f"| kernel | MFMA busy (of {simds} SIMDs x active cycles) | bf16 MFMA GFLOP per dispatch |")
        print("|---|---:|---:|")
        for k, d in sorted(rows, key=lambda r: -r[1]["SQ_VALU_MFMA_BUSY_CYCLES"]):
            busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / 8 * simds)
            fl = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
            print(f"| `{_short(k)}` | {busy:.3f} | {fl * 512 / 1e9:.1f} |" if fl is not None else
                  f"| `{_short(k)}` | {busy:.3f} | - |")


# ---------------------------------------------------------------- workloads ----
def cnp_bench(wl, steps, warmup, theta_bf16=False):
    """Workload 2: CNP forward (G in bf16) and backward on independent blocks; theta_bf16:
    the same draws stored as bf16 (then Q is exact in bf16 and the kernels skip its lo part)."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd import workloads as WL
    theta, dg = WL.make_cnp_inputs(wl.nblocks, wl.b, wl.theta_std, seed=WL.BASE_SEED + wl.key)
    th = torch.from_numpy(theta).cuda()
    if theta_bf16:
        th = th.to(torch.bfloat16)
    dgt = torch.from_numpy(dg).cuda()
    del theta, dg
    g = torch.empty((wl.nblocks, wl.b, wl.b), dtype=torch.bfloat16, device="cuda")
    dth = torch.empty(th.shape, dtype=torch.float32, device="cuda")  # dtheta is float32 whatever theta is
    q = B.qsave_like(th, wl.b)  # the forward keeps Q's planes; the backward reads them
    res, per = {}, {}
    for name, fn in (("fwd", lambda: B.poetx_cnp(B.POETX_CNP_FWD, th, wl.b, g=g, qsave=q)),
                     ("bwd", lambda: B.poetx_cnp(B.POETX_CNP_BWD, th, wl.b, dg=dgt, dtheta=dth, qsave=q))):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            fn()
            _sync()
        for _ in range(warmup):
            fn()
        _sync()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i].record()
            fn()
        ev[steps].record()
        _sync()
        res[name] = (time.perf_counter() - t0) * 1e3 / steps
        per[name] = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    b, n = wl.b, wl.nblocks
    # method flops: forward 2 b^3-products (Horner), backward 6 (each 2 b^3)
    f_fwd, f_bwd = 4.0 * b ** 3 * n, 12.0 * b ** 3 * n
    p = b * (b - 1) // 2
    y_fwd, y_bwd = n * (4 * p + 2 * b * b), n * (4 * b * b + 8 * p)
    ms = res["fwd"] + res["bwd"]
    del th, dgt, g, dth, q
    torch.cuda.empty_cache()
    return {
        "metric": "CNP fwd+bwd blocks/s (4096 x b=256)", "value": n / (ms * 1e-3), "unit": "blocks/s",
        "saved_q": True, "theta_dtype": "bf16" if theta_bf16 else "f32",
        "ms_per_step": ms, "fwd_ms": res["fwd"], "bwd_ms": res["bwd"],
        "fwd_ms_median": statistics.median(per["fwd"]), "bwd_ms_median": statistics.median(per["bwd"]),
        "config": {"workload": wl.name, "nblocks": n, "b": b},
        "fwd_frac_mfma_method_flops": f_fwd / (res["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "bwd_frac_mfma_method_flops": f_bwd / (res["bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "fwd_frac_hbm": y_fwd / (res["fwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "bwd_frac_hbm": y_bwd / (res["bwd"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "floor_ms_single_pass": (max(f_fwd / 2.5e15, y_fwd / 8e12) + max(f_bwd / 2.5e15, y_bwd / 8e12)) * 1e3,
    }


def layer_summary(wl, steps, warmup):
    """One layer workload's variants, for the lines beside the head workload."""
    from orthogonal_reparameterized_amd import workloads as WL
    inputs = WL.make_layer_inputs(wl)
    out = {"config": {"workload": wl.name, "n_tokens": wl.n_tokens, "d_in": wl.d_in, "d_out": wl.d_out,
                      "b": wl.b, "weight": wl.w}}
    for variant in wl.variants:
        keep_wt = variant == "fast" and wl.w == "bf16"
        v, ph, _ = run_variant(wl, inputs, variant, steps, warmup, keep_wt=keep_wt)
        v["dominant"] = {k: ph[k] for k in ("gemm_nt", "gemm_nn") if k in ph}
        out[variant] = v
    return out


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mem", action="store_true")
    ap.add_argument("--only-head", action="store_true",
                    help="only the head workload's headline variant (and mem unless --no-mem)")
    ap.add_argument("--no-wt", action="store_true", help="fast variant without the W'^T copy")
    ap.add_argument("--steps-only", action="store_true",
                    help="profiling runs: only the layer steps (no cold-cache pass, peaks, merge, fold, Adam)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps before the warm-up (seconds; 0 for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--theta-bf16", action="store_true", help="workload 2 with theta stored in bf16")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DB [BENCH_JSON]")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DB")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DB")
    args = ap.parse_args()
    SETTLE_S = args.settle_s
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace[:2])
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters[:5])
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens with an all-reduce of dtheta).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    from orthogonal_reparameterized_amd import workloads as WL

    wl = WL.WORKLOADS[args.workload]
    if wl.nblocks:
        r = cnp_bench(wl, args.steps, args.warmup, theta_bf16=args.theta_bf16)
        r.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                  "scaling": "weak", "vs_baseline": None, "dtype": "f32 (split-bf16 MFMA)", "data": "synthetic"})
        print(json.dumps(r))
        return
    inputs = WL.make_layer_inputs(wl)
    n = wl.n_tokens
    variants, phases = {}, {}
    head = "fast" if "fast" in wl.variants else "mem"
    cold = None
    for variant in wl.variants:
        if variant == "mem" and args.no_mem and "fast" in wl.variants:
            continue
        # the headline fast variant also keeps W'^T from the merge (one more weight copy; the
        # backward's product then reads W' k-contiguous) and the gathered input X~
        keep_wt = variant == "fast" and wl.w == "bf16" and not args.no_wt
        v, ph, c = run_variant(wl, inputs, variant, args.steps, args.warmup, keep_wt=keep_wt,
                               cold_steps=5 if variant == head and not args.steps_only else 0)
        variants[variant], phases[variant] = v, ph
        if variant == head:
            cold = c
    if not args.only_head and "fast" in wl.variants:
        # the pages' own fast variant keeps only B; and the literal chain without the two
        # activation permutations
        v, ph, _ = run_variant(wl, inputs, "fast", args.steps, args.warmup, keep_wt=False, keep_x=False)
        variants["fast_pages"], phases["fast_pages"] = v, ph
        v, ph, _ = run_variant(wl, inputs, "fast", args.steps, args.warmup,
                               keep_wt=wl.w == "bf16" and not args.no_wt, perms=False)
        variants["fast_null_perm"], phases["fast_null_perm"] = v, ph

    ms = variants[head]["ms_per_step"]
    dom = phases[head].get(DOMINANT + " (timed steps)")
    if args.steps_only:
        print(json.dumps({"metric": METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                          "step_ms": variants[head]["step_ms"], "variants": variants, "phases": phases,
                          "config": {"workload": wl.name, "variant": head},
                          "roofline": {"kernel": DOMINANT, "avg_launch_ms": dom["avg_ms"] if dom else None}}))
        return
    peaks = measured_peaks(wl)
    roof = None
    if dom:
        flops_launch = 2.0 * n * wl.d_in * wl.d_out
        achieved = flops_launch / (dom["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic(DOMINANT, wl.key),
                "kernel": DOMINANT, "avg_launch_ms": dom["avg_ms"],
                "launches": int(round(dom["launches_per_step"] * args.steps)),
                "algorithmic_flops_per_launch": flops_launch,
                "measured_peak": peaks["library_gemm_TF_s"],
                "frac_of_measured_peak": achieved / peaks["library_gemm_TF_s"],
                "timing": "dispatch-bound start/stop events on this kernel's launches inside the timed steps"}
    for ph in list(phases.values()) + ([cold] if cold else []):
        for e in ph.values():
            if "gbs" in e:
                e["frac_hbm_measured_copy"] = e["gbs"] / peaks["copy_GB_s"]
    merge_ms, merge_gbs = merge_time_ms(wl, inputs)
    merge_t_ms, merge_t_gbs = merge_time_ms(wl, inputs, with_t=True) if wl.w == "bf16" else (None, None)
    out = {
        "metric": METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.act, "data": "synthetic",
        "config": {"workload": wl.name, "n_tokens": n, "d_in": wl.d_in, "d_out": wl.d_out, "b": wl.b,
                   "variant": head, "activation_permutations": wl.perms, "weight": wl.w},
        "roofline": roof,
        "step_ms": variants[head]["step_ms"],
        "variants": variants,
        "phases": phases,
        "phases_cold_cache": cold,
        "measured_peaks": peaks,
        "merge_per_phase": {"ms": merge_ms, "GB_s": merge_gbs,
                            "with_transpose_ms": merge_t_ms, "with_transpose_GB_s": merge_t_gbs,
                            "fold_ms": fold_time_ms(wl, inputs)},
        "optimizer_per_step": adam_time_ms(wl),
    }
    del inputs
    if not args.only_head:
        others = {}
        for key in (1, 4, 5, 6):
            if key != args.workload:
                others[str(key)] = layer_summary(WL.WORKLOADS[key], max(5, args.steps // 2), 3)
        others["2"] = cnp_bench(WL.WORKLOADS[2], max(5, args.steps // 2), 2)
        others["2_bf16_theta"] = cnp_bench(WL.WORKLOADS[2], max(5, args.steps // 2), 2, theta_bf16=True)
        out["other_workloads"] = others
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, WL.make_layer_inputs(wl))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
