"""Benchmark of the `blr` layer's forward + backward on one MI355X.

One step = blr_forward + blr_backward (all steps of the layer) over one
batch of seeded synthetic input that is already resident in HBM. Default
workload: the attention-projection layer M=8192 tokens, d_in=d_out=4096,
r=512. Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

# MI355X published peaks
PEAK_F16_TFLOPS = 2516.6  # dense f16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0     # HBM3E
RIDGE = PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte


def kernel_work(name: str, w: synth.Workload, keep_c: bool = False) -> tuple[float, float]:
    """Algorithmic (bytes, flops) of one launch of a kernel: the bytes each
    kernel must move between HBM and the chip at minimum (f32 activations in
    and out once, the 1-bit sign bitmap once, the per-column scales) and the
    MFMA flops of its contraction."""
    M, di, do, r = w.M, w.d_in, w.d_out, w.r
    f32 = 4
    if name == "gemm_f1_xg_sv":      # read x, write tape a; bitmap of S_V
        return M * (di + r) * f32 + r * di / 8 + di * f32, 2.0 * M * r * di
    if name == "gemm_f2_al_sut":     # read a, write y (and the c tape); bitmap of S_U
        return M * (r + (2 if keep_c else 1) * do) * f32 + do * r / 8 + (r + do) * f32, 2.0 * M * do * r
    if name == "gemm_dh_recompute_c":  # read a and dy; dh partials are negligible
        return M * (r + do) * f32 + do * r / 8 + r * f32, 2.0 * M * do * r
    if name == "gemm_b1_dyh_su":     # read dy and a, write db
        return M * (do + 2 * r) * f32 + r * do / 8 + do * f32, 2.0 * M * r * do
    if name == "gemm_b1_dh_fused":   # read dy and a, write db; B1 plus c recomputed for dh (two contractions)
        return M * (do + 2 * r) * f32 + 2 * r * do / 8 + do * f32 + r * f32, 4.0 * M * r * do
    if name == "gemm_b2_dbl_svt":    # read db and x, write dx
        return M * (r + 2 * di) * f32 + di * r / 8 + (r + di) * f32, 2.0 * M * di * r
    if name == "gemm_f2_two_paths":  # the two-path layer's F2 (the paths' ranks add up to r)
        return kernel_work("gemm_f2_al_sut", w)
    if name == "gemm_b2_two_paths":  # the two-path layer's B2
        return kernel_work("gemm_b2_dbl_svt", w)
    if name == "gemm_sign_grads":    # read dy, a, x, db; write G_U, G_V
        return M * (do + di + 2 * r) * f32 + (do + di) * r * f32, 2.0 * M * r * (do + di)
    if name == "sign_grads_zero":    # zero G_U, G_V before the token ranges add into them
        return (do + di) * r * f32, 0.0
    if name == "colsum_dy_c":        # read dy and c
        return 2.0 * M * do * f32, 2.0 * M * do
    if name == "transpose_bits":     # one bitmap in, its transpose out (average of U and V)
        return 2 * r * (di + do) / 2 / 8, 0.0
    if name == "colsum_finish":      # read the column partials of dh, dl, dg
        mt = -(-M // 64)  # every producer uses 64-token tiles; fused dh at r = 512: two rank tiles
        rows_h = 2 * mt if (not keep_c and r == 512) else mt
        return (rows_h * do + mt * (r + di)) * f32, 0.0
    if name == "expand_signs":       # per launch: one bitmap in, one f16 plane out (average of U and V)
        rows = (di + do) / 2
        return rows * (r / 8 + r * 2), 0.0
    return 0.0, 0.0


def source_digest() -> str:
    """sha256 (first 16 hex digits) of the HIP library's sources: a profile
    summary records the digest of the kernels it measured."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "binary_rank_linear_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from profiles/hbm_traffic_<workload>.md
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated against a copy kernel), or
    None when there is no summary or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest, val = None, None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("source_digest:"):
                digest = line.split(":", 1)[1].strip()
            elif line.startswith(f"traffic_bytes {kernel}:"):
                val = int(line.split(":", 1)[1])
    return val if digest == source_digest() else None


def gen_inputs(w: synth.Workload, dev):
    import torch
    d = synth.inputs(w)
    t = {}
    for k, v in d.items():
        if v.dtype == np.uint32:
            v = v.view(np.int32)
        t[k] = torch.from_numpy(v).to(dev)
    return d, t


def cpu_baseline(w: synth.Workload, d: dict, target_s: float = 12.0) -> dict:
    """The f64 oracle, as it stands, on the first tokens of the same inputs:
    a 1024-token calibration run, then a sample sized to about target_s."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        oracle.forward(d["x"][:n], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"], tape=False)
        oracle.backward(d["x"][:n], d["dy"][:n], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
        return time.perf_counter() - t0

    n = min(w.M, 1024)
    dt = run(n)
    if dt < 0.4 * target_s and n < w.M:
        n = int(min(w.M, max(n, n * target_s / dt)))
        n = max(64, (n // 64) * 64)
        dt = run(n)
    reps = 1
    if n == w.M and dt < 0.4 * target_s:
        # the whole workload is the sample: repeat it for a steadier figure
        reps = max(1, int(target_s / max(dt, 1e-3)))
        dt = sum(run(n) for _ in range(reps)) / reps
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {n} of {w.M} tokens of the same workload, fwd+bwd in f64, {dt:.2f} s per pass, "
                      f"mean of {reps} pass(es)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=synth.HEADLINE, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keep-c", action="store_true",
                    help="store the f32 c tape in the forward (the page's layout) instead of recomputing c")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the run, copy a buffer of this many MiB three times with torch (a plain copy "
                         "kernel of known traffic, for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer's data-parallel split and its "
              "gradient all-reduce are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    import binary_rank_linear_amd as blr

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    blr.load()
    if not blr.device_supported(0):
        raise SystemExit("cuda:0 is not gfx950")
    print(f"# workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    d, t = gen_inputs(w, dev)
    M, di, do, r = w.M, w.d_in, w.d_out, w.r
    y = torch.empty((M, do), dtype=torch.float32, device=dev)
    ta = torch.empty((M, r), dtype=torch.float32, device=dev)
    tc = torch.empty((M, do), dtype=torch.float32, device=dev) if args.keep_c else None
    dx = torch.empty((M, di), dtype=torch.float32, device=dev)
    dh = torch.zeros(do, dtype=torch.float32, device=dev)
    dl = torch.zeros(r, dtype=torch.float32, device=dev)
    dg = torch.zeros(di, dtype=torch.float32, device=dev)
    ws = blr.workspace(M, di, do, r, dev)

    def fwd():
        blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], y=y, tape_a=ta, tape_c=tc, ws=ws)

    def bwd():
        blr.blr_backward(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc, w.gscale,
                         dh=dh, dl=dl, dg=dg, dx=dx, ws=ws)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # forward and backward alone (context)
    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    fwd_ms = timed(fwd, args.steps)
    bwd_ms = timed(bwd, args.steps)

    # per-kernel durations: HIP events the library records around each of its
    # launches, on the launch stream, over a second timed region of K steps
    blr.blr_profile_enable(args.steps * 16)
    blr.blr_profile_reset()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = blr.blr_profile_read()
    blr.blr_profile_enable(0)
    kernels = {}
    for name, (count, tot_ms) in prof.items():
        avg_us = 1000.0 * tot_ms / count
        nbytes, flops = kernel_work(name, w, args.keep_c)
        kernels[name] = {"launches_per_step": count / args.steps, "avg_us": round(avg_us, 3),
                         "gbs": round(nbytes / (avg_us * 1e-6) / 1e9, 1) if nbytes else None,
                         "tflops": round(flops / (avg_us * 1e-6) / 1e12, 1) if flops else None}
    dom = max(prof, key=lambda k: prof[k][1])
    nbytes, flops = kernel_work(dom, w, args.keep_c)
    avg_s = prof[dom][1] / prof[dom][0] / 1000.0
    if flops and flops / nbytes > RIDGE:
        roof = {"bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["avg_us"] = round(avg_s * 1e6, 3)

    # sign gradients (blr_backward_signs, not part of the headline step):
    # the duration of their contraction over the same K backward calls
    gu = torch.empty((do, r), dtype=torch.float32, device=dev)
    gv = torch.empty((di, r), dtype=torch.float32, device=dev)
    blr.blr_profile_enable(args.steps * 16)
    blr.blr_profile_reset()
    for _ in range(args.steps):
        blr.blr_backward_signs(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], ta, tc, w.gscale,
                               dh=dh, dl=dl, dg=dg, dx=dx, grad_u=gu, grad_v=gv, ws=ws)
    torch.cuda.synchronize()
    sprof = blr.blr_profile_read()
    blr.blr_profile_enable(0)
    sign = None
    if "gemm_sign_grads" in sprof:
        cnt, tot = sprof["gemm_sign_grads"]
        s_us = 1000.0 * tot / cnt
        sb, sf = kernel_work("gemm_sign_grads", w)
        sign = {"avg_us": round(s_us, 3), "tflops": round(sf / (s_us * 1e-6) / 1e12, 1),
                "frac_f16_peak": round(sf / (s_us * 1e-6) / 1e12 / PEAK_F16_TFLOPS, 4),
                "gbs": round(sb / (s_us * 1e-6) / 1e9, 1)}

    # the fused layer of two paths of half the rank each (same MFMA work as
    # the one-path step): blr_forward_paths + blr_backward_paths
    multi = None
    if r % 256 == 0:
        P, rp = 2, r // 2
        dp = synth.custom_paths(M, di, do, rp, P, seed=9100, dy_sigma=w.dy_sigma, l_hi=w.l_hi)
        tp = {k: torch.from_numpy(np.ascontiguousarray(dp[k].view(np.int32) if dp[k].dtype == np.uint32 else dp[k]))
              .to(dev) for k in ("bits_u", "bits_v", "h", "l", "g")}
        yp = torch.empty((M, do), dtype=torch.float32, device=dev)
        tap = torch.empty((M, P * rp), dtype=torch.float32, device=dev)
        dhp = torch.zeros((P, do), dtype=torch.float32, device=dev)
        dlp = torch.zeros((P, rp), dtype=torch.float32, device=dev)
        dgp = torch.zeros((P, di), dtype=torch.float32, device=dev)
        wsp = blr.workspace_paths(M, di, do, rp, P, dev)

        def step_p():
            blr.blr_forward_paths(t["x"], tp["bits_u"], tp["bits_v"], tp["h"], tp["l"], tp["g"], y=yp, tape_a=tap,
                                  ws=wsp)
            blr.blr_backward_paths(t["x"], t["dy"], tp["bits_u"], tp["bits_v"], tp["h"], tp["l"], tp["g"], tap,
                                   w.gscale, dh=dhp, dl=dlp, dg=dgp, dx=dx, ws=wsp)

        for _ in range(max(args.warmup, 1)):
            step_p()
        torch.cuda.synchronize()
        ms_p = timed(step_p, args.steps)
        fl = 6.0 * M * P * rp * (di + do)
        multi = {"paths": P, "rank_per_path": rp, "ms_per_step": round(ms_p, 5),
                 "tokens_per_s": round(M / (ms_p / 1000.0), 1), "tflops_metric": round(fl / (ms_p / 1000.0) / 1e12, 2)}
        del tp, yp, tap, dhp, dlp, dgp, wsp

    tokens_s = M / (ms / 1000.0)
    tf_metric = w.flops_metric() / (ms / 1000.0) / 1e12
    tf_mfma = w.flops_mfma() / (ms / 1000.0) / 1e12
    out = {
        "metric": "blr fwd+bwd tokens/s and TFLOP/s (% of f16 MFMA peak) at d=4096, r=512",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "d_in": di, "d_out": do, "r": r, "gscale": w.gscale,
                   "accumulate": "f32", "paths": 1, "c_tape": "f32" if args.keep_c else "recomputed"},
        "tflops_metric": round(tf_metric, 2),
        "pct_f16_peak_metric": round(100 * tf_metric / PEAK_F16_TFLOPS, 2),
        "tflops_mfma": round(tf_mfma, 2),
        "pct_f16_peak_mfma": round(100 * tf_mfma / PEAK_F16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "kernels": kernels,
        "roofline": roof,
        "sign_grads": sign,
        "multi_path": multi,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("# oracle CPU baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
