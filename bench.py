#!/usr/bin/env python3
"""POET-X layer forward+backward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3]

A step is one pass of the layer's hot path on one batch: CNP forward of G_R and
G_P, the layer forward, the layer backward (which ends with the CNP backward).
The permutation merge runs once per inner phase, before the timed region, and
is timed separately.  Inputs are seeded synthetic data resident in HBM before
timing starts.  Prints ONE JSON line.

Extra modes used to make the committed profile summaries:
    --copy-calibration   time a plain 1 GiB device copy (the HBM counter calibration)
    --no-cpu             skip the CPU-oracle baseline leg
    --summarize-trace DB [JSON]      markdown kernel table from a rocprofv3 --kernel-trace database
                                     (with the traced run's JSON line: dominant kernel trace vs events)
    --summarize-counters F W CF CW   HBM traffic of the dominant kernel from four rocprofv3 --pmc
                                     databases (FETCH_SIZE, WRITE_SIZE; then the same two counters
                                     taken on --copy-calibration)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "POET-X layer fwd+bwd tokens/s (4096², b=256) + % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
DOMINANT = "gemm_nt"


def algorithmic(wl, variant, n):
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
        add("permute_cols", 0, 2 * n * di * ae)
        add("block_apply", 2.0 * n * di * b, 2 * n * di * ae + g_bytes_r)
        add("gemm_nt", 2.0 * n * di * do, n * di * ae + do * di * we + n * do * ae)
    # fast keeps the forward's X~ for dG_R (the gather above writes it): no second gather
    add("block_apply", 2.0 * n * do * b, 2 * n * do * ae + g_bytes_p)            # Z~ = B G_P
    add("permute_cols", 0, 2 * n * do * ae)                                       # scatter Z
    add("permute_cols", 0, 2 * n * do * ae)                                       # gather dZ
    add("block_apply_t", 2.0 * n * do * b, 2 * n * do * ae + g_bytes_p)          # dB
    add("block_grad", 2.0 * n * do * b, 2 * n * do * ae)                          # dG_P
    add("gemm_nn", 2.0 * n * di * do, n * do * ae + do * di * we + n * di * ae)   # dA
    add("block_apply_t", 2.0 * n * di * b, 2 * n * di * ae + g_bytes_r)          # dX~
    add("permute_cols", 0, 2 * n * di * ae)                                       # scatter dX
    add("block_grad", 2.0 * n * di * b, 2 * n * di * ae)                          # dG_R
    # CNP, both sides (nb blocks): the forward chain G = (((Q+2I)Q+2I)Q+2I)Q + I runs 3
    # float32-accurate b^3 products (2 b^3 flops each); the backward 8 in one fused launch
    # when the blocks fill the GPU, else 3 + 3 in two chain launches.
    # Bytes are the method's minimum: theta in and G out (forward), theta and dG in and
    # dtheta out (backward, split over its two launches); the unpack and pack launches
    # carry the theta / dtheta side.
    nb = nr + np_
    p, bb = b * (b - 1) // 2, b * b
    add("unpack_skew", 0, 2 * nb * 4 * p)
    add("cnp_fwd_chain", 6.0 * b ** 3 * nb, nb * ae * bb)
    if nb * (b // 64) >= 4 * 256:
        add("cnp_bwd_fused", 16.0 * b ** 3 * nb, nb * 4 * bb)   # 8 products in one launch
    else:
        add("cnp_bwd_chain_a", 6.0 * b ** 3 * nb, nb * 4 * bb)  # few blocks: two launches
        add("cnp_bwd_chain_b", 6.0 * b ** 3 * nb, 0)
    add("pack_skew_grad", 0, nb * 4 * p)
    return ops


def step_flops(wl, variant, n):
    return sum(f for f, _ in algorithmic(wl, variant, n).values())


def layer_roofline_ms(wl, variant, n):
    """Sum over kernels of max(flops / MFMA peak, bytes / HBM peak).  The CNP products
    are float32-accurate through three bf16 MFMA passes, so they count 3x against the
    bf16 peak; everything else runs one bf16 pass per product."""
    t = 0.0
    for name, (f, y) in algorithmic(wl, variant, n).items():
        passes = 3 if name.startswith("cnp_") else 1
        t += max(passes * f / (PEAK_BF16_TFLOPS * 1e12), y / (PEAK_HBM_GBS * 1e9))
    return t * 1e3


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
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.poetx_fold(st.layer, w_out)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def adam_time_ms(wl, reps=20):
    """poetx_adam_step over the layer's packed theta (both sides), float32 state."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    n = (wl.d_in // wl.b + wl.d_out // wl.b) * (wl.b * (wl.b - 1) // 2)
    th = torch.zeros(n, device="cuda")
    g, m, v = torch.randn(n, device="cuda"), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    B.poetx_adam_step(th, g, m, v, lr=1e-3, step=1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(reps):
        B.poetx_adam_step(th, g, m, v, lr=1e-3, step=t + 2)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": ms, "params": n, "GB_s": 7 * 4 * n / (ms * 1e-3) / 1e9}


def time_steps(st, steps, warmup):
    import torch
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def profile_steps(st, steps):
    """Per-kernel-label launch counts and average durations (HIP events on the
    library's launch stream, recorded around each launch)."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    B.prof_read()  # clear
    B.prof_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    B.prof_enable(False)
    rec = B.prof_read()
    return {k: (n / steps, ms / n) for k, (n, ms) in rec.items()}, wall


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
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.poetx_merge_perm(w, pout, pin, s, out, so, ot)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = (4 if with_t else 2) * w.numel() * w.element_size()
    return ms, nbytes / (ms * 1e-3) / 1e9


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


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GB_s_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))


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


def summarize_trace(db, bench_json=None):
    """Markdown kernel table of a --kernel-trace database; with the JSON line that the
    traced bench.py run printed, also the dominant kernel's trace average next to the
    event-timed average that run reported (the last launches are the event-timed ones)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                       "sum(duration) from kernels group by name order by sum(duration) desc").fetchall()
    tot = sum(r[5] for r in rows)
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, n, avg, mn, mx, sm in rows:
        short = name.replace("(poetx::KArgs)", "").replace("poetx::", "")[:90]
        print(f"| `{short}` | {n} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | {100 * sm / tot:.1f}% |")
    if bench_json:
        line = [ln for ln in open(bench_json) if ln.startswith("{")][-1]
        d = json.loads(line)
        roof = d.get("roofline") or {}
        if "phases" not in d:  # the CNP microbenchmark: no per-label phases
            print()
            print(f"bench.py in this run: forward {d['fwd_ms']:.3f} ms, backward {d['bwd_ms']:.3f} ms per call "
                  f"over {d['config']['nblocks']} blocks of b = {d['config']['b']}: "
                  f"{d['value'] / 1e3:.0f} K blocks/s.")
            return
        ph = d["phases"][d["config"]["variant"]][roof["kernel"]]
        n_ev = int(round(ph["launches_per_step"] * d["steps"]))
        if roof["kernel"] == "gemm_nt" and d["variants"][d["config"]["variant"]].get("w_merged_t"):
            n_ev *= 2  # the backward product runs the same kernel (on W'^T) in the fast variant
        sym = KERNEL_SYMBOL[roof["kernel"]].replace(" ", "")
        durs = [r[1] for r in con.execute("select name, duration from kernels order by start")
                if sym in r[0].replace(" ", "")]
        last = durs[-n_ev:]
        print()
        print(f"Dominant kernel `{roof['kernel']}` (`{sym}`) in this run: trace average over all "
              f"{len(durs)} launches {sum(durs) / len(durs) / 1e3:.1f} us, over the last {len(last)} "
              f"(the event-timed ones) {sum(last) / len(last) / 1e3:.1f} us; bench.py's event-timed "
              f"average {roof['avg_launch_ms'] * 1e3:.1f} us -> {roof['achieved']:.0f} TFLOP/s, "
              f"frac {roof['frac']:.3f}; step {d['ms_per_step']:.4f} ms, {d['value'] / 1e6:.3f} M tokens/s.")


def summarize_counters(fetch_db, write_db, copy_fetch_db, copy_write_db, label=DOMINANT):
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        return con.execute("select kernel_name, count(*), avg(value) from counters_collection "
                           "where counter_name = ? group by kernel_name", (counter,)).fetchall()

    def pick(rows, match):
        for name, n, v in rows:
            if match in name.replace(" ", ""):
                return n, v
        raise SystemExit(f"no kernel matching {match}")

    copy_kib = float(1 << 30) / 1024
    _, cf = pick(per_kernel(copy_fetch_db, "FETCH_SIZE"), "copyBuffer")
    _, cw = pick(per_kernel(copy_write_db, "WRITE_SIZE"), "copyBuffer")
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    sym = KERNEL_SYMBOL[label]
    nf, f = pick(per_kernel(fetch_db, "FETCH_SIZE"), sym)
    nw, w = pick(per_kernel(write_db, "WRITE_SIZE"), sym)
    print(f"kernel_label = {label}")
    print(f"kernel_symbol_match = {sym}")
    print(f"dispatches_fetch = {nf}")
    print(f"dispatches_write = {nw}")
    print(f"fetch_kib_per_dispatch_raw = {f:.1f}")
    print(f"write_kib_per_dispatch_raw = {w:.1f}")
    print(f"copy_fetch_kib_raw = {cf:.1f}  (1 GiB copy reads {copy_kib:.0f} KiB)")
    print(f"copy_write_kib_raw = {cw:.1f}  (1 GiB copy writes {copy_kib:.0f} KiB)")
    print(f"fetch_scale = {f_scale:.4f}")
    print(f"write_scale = {w_scale:.4f}")
    print(f"traffic_bytes_per_launch = {(f * f_scale + w * w_scale) * 1024:.0f}")
    print(f"kernel_sources = {' + '.join(os.path.relpath(f, ROOT) for f in KERNEL_SOURCES)}")
    print(f"kernel_source_sha = {kernel_source_sha()}")


def cnp_bench(wl, steps, warmup):
    """Workload 2: CNP forward (G in bf16) and backward on independent blocks."""
    import torch
    from orthogonal_reparameterized_amd import binding as B
    from orthogonal_reparameterized_amd import workloads as WL
    theta, dg = WL.make_cnp_inputs(wl.nblocks, wl.b, wl.theta_std, seed=WL.BASE_SEED + wl.key)
    th = torch.from_numpy(theta).cuda()
    dgt = torch.from_numpy(dg).cuda()
    del theta, dg
    g = torch.empty((wl.nblocks, wl.b, wl.b), dtype=torch.bfloat16, device="cuda")
    dth = torch.empty_like(th)
    res = {}
    for name, fn in (("fwd", lambda: B.poetx_cnp(B.POETX_CNP_FWD, th, wl.b, g=g)),
                     ("bwd", lambda: B.poetx_cnp(B.POETX_CNP_BWD, th, wl.b, dg=dgt, dtheta=dth))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) * 1e3 / steps
    b, n = wl.b, wl.nblocks
    # float32-equivalent flops: forward 2 b^3-products, backward 6 (each 2 b^3)
    f_fwd, f_bwd = 4.0 * b ** 3 * n, 12.0 * b ** 3 * n
    ms = res["fwd"] + res["bwd"]
    out = {
        "metric": "CNP fwd+bwd blocks/s (4096 x b=256)", "value": n / (ms * 1e-3), "unit": "blocks/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (split-bf16 MFMA)", "data": "synthetic",
        "config": {"workload": wl.name, "nblocks": n, "b": b},
        "fwd_ms": res["fwd"], "bwd_ms": res["bwd"],
        "fwd_tflops_f32_equiv": f_fwd / (res["fwd"] * 1e-3) / 1e12,
        "bwd_tflops_f32_equiv": f_bwd / (res["bwd"] * 1e-3) / 1e12,
        # three bf16 MFMA passes per float32-accurate product
        "roofline": {"bound": "mfma", "achieved": 3 * (f_fwd + f_bwd) / (ms * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": 3 * (f_fwd + f_bwd) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": None, "kernel": "cnp (all launches, bf16 MFMA passes)"},
    }
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mem", action="store_true")
    ap.add_argument("--no-wt", action="store_true", help="fast variant without the W'^T copy")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DB [BENCH_JSON]")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DB")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace[:2])
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens with an all-reduce of dtheta).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from orthogonal_reparameterized_amd import workloads as WL
    from orthogonal_reparameterized_amd.step import LayerStep

    wl = WL.WORKLOADS[args.workload]
    if wl.nblocks:
        cnp_bench(wl, args.steps, args.warmup)
        return
    inputs = WL.make_layer_inputs(wl)
    n = wl.n_tokens
    variants = {}
    phases = {}
    for variant in wl.variants:
        if variant == "mem" and args.no_mem and "fast" in wl.variants:
            continue
        # the fast variant also keeps W'^T from the merge (one more weight copy, the
        # backward's product then reads W' k-contiguous); mem stays memory-lean
        keep_wt = variant == "fast" and wl.w == "bf16" and not args.no_wt
        st = LayerStep(wl, inputs, variant, transposed_weight=keep_wt)
        ms = time_steps(st, args.steps, args.warmup)
        prof, prof_wall = profile_steps(st, args.steps)
        alg = algorithmic(wl, variant, n)
        variants[variant] = {"ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3), "w_merged_t": keep_wt,
                             "kept_x": st.saved_x is not None,
                             "layer_roofline_ms": layer_roofline_ms(wl, variant, n),
                             "roofline_frac": layer_roofline_ms(wl, variant, n) / ms,
                             "ms_per_step_with_event_hooks": prof_wall}
        ph = {}
        for name, (launches, avg_ms) in sorted(prof.items()):
            ph[name] = {"launches_per_step": launches, "avg_ms": avg_ms}
            if name in alg:
                f, y = alg[name]
                per = launches if launches else 1
                ph[name]["tflops"] = f / per / (avg_ms * 1e-3) / 1e12
                ph[name]["gbs"] = y / per / (avg_ms * 1e-3) / 1e9
        phases[variant] = ph
        del st
        torch.cuda.empty_cache()

    head = "fast" if "fast" in variants else "mem"
    ms = variants[head]["ms_per_step"]
    dom = phases[head].get(DOMINANT)
    roof = None
    if dom:
        flops_launch = 2.0 * n * wl.d_in * wl.d_out
        achieved = flops_launch / (dom["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic(DOMINANT, wl.key),
                "kernel": DOMINANT, "avg_launch_ms": dom["avg_ms"],
                "algorithmic_flops_per_launch": flops_launch}
    merge_ms, merge_gbs = merge_time_ms(wl, inputs)
    merge_t_ms, merge_t_gbs = merge_time_ms(wl, inputs, with_t=True) if wl.w == "bf16" else (None, None)
    out = {
        "metric": METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.act, "data": "synthetic",
        "config": {"workload": wl.name, "n_tokens": n, "d_in": wl.d_in, "d_out": wl.d_out, "b": wl.b,
                   "variant": head, "activation_permutations": wl.perms, "weight": wl.w},
        "roofline": roof,
        "variants": variants,
        "phases": phases,
        "merge_per_phase": {"ms": merge_ms, "GB_s": merge_gbs,
                            "with_transpose_ms": merge_t_ms, "with_transpose_GB_s": merge_t_gbs,
                            "fold_ms": fold_time_ms(wl, inputs)},
        "optimizer_per_step": adam_time_ms(wl),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, inputs)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
