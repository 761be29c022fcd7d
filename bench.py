"""Benchmark of the `blr` layer's forward + backward on one MI355X.

One step = blr_forward + blr_backward (all steps of the layer) over one
batch of seeded synthetic input that is already resident in HBM. The
headline workload is the attention-projection layer M=8192 tokens,
d_in=d_out=4096, r=512; the other workloads (the tiny layer, the 2048-token
windows layer, the MLP up+down pair timed as one step, the ragged
30000-token layer) are measured the same way and reported under "configs"
in the same JSON line. Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--configs all|none] [--no-cpu-baseline] [--keep-c]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
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

# the MLP up + down pair is one bench line: two independent layers
PAIR = ("mlp_up_8192x4096x12288_r1024", "mlp_down_8192x12288x4096_r1024")
PAIR_NAME = "mlp_pair_8192x4096x12288_r1024"


def kernel_work(name: str, w: synth.Workload, keep_c: bool = False) -> tuple[float, float, float]:
    """Algorithmic (bytes, flops, executed flops) of one launch of a kernel.

    bytes: what the kernel must move between HBM and the chip at minimum
    (f32 activations in and out once, the 1-bit sign bitmaps once, the
    per-column scales). flops: the method's own work in that launch (its
    contraction, or its column reduction). executed flops: what the launch
    performs, which differs where c is recomputed for dh (the page reads c
    from its tape; recomputing it is an implementation choice, not the
    method's work)."""
    M, di, do, r = w.M, w.d_in, w.d_out, w.r
    f32 = 4
    if name == "gemm_f1_xg_sv":      # read x, write tape a; bitmap of S_V
        b, f = M * (di + r) * f32 + r * di / 8 + di * f32, 2.0 * M * r * di
        return b, f, f
    if name == "gemm_f2_al_sut":     # read a, write y (and the c tape); bitmap of S_U
        b, f = M * (r + (2 if keep_c else 1) * do) * f32 + do * r / 8 + (r + do) * f32, 2.0 * M * do * r
        return b, f, f
    if name == "gemm_dh_recompute_c":  # read a and dy; the method's dh is the column sum of dy.c
        return M * (r + do) * f32 + do * r / 8 + r * f32, 2.0 * M * do, 2.0 * M * do * r + 2.0 * M * do
    if name == "gemm_b1_dyh_su":     # read dy and a, write db
        b, f = M * (do + 2 * r) * f32 + r * do / 8 + do * f32, 2.0 * M * r * do + 2.0 * M * r
        return b, f, f
    if name == "gemm_b1_dh_fused":   # read dy and a, write db; B1, the dl and dh column sums, c recomputed
        b = M * (do + 2 * r) * f32 + 2 * r * do / 8 + do * f32 + r * f32
        f = 2.0 * M * r * do + 2.0 * M * r + 2.0 * M * do
        return b, f, f + 2.0 * M * r * do
    if name == "gemm_b2_dbl_svt":    # read db and x, write dx
        b, f = M * (r + 2 * di) * f32 + di * r / 8 + (r + di) * f32, 2.0 * M * di * r + 2.0 * M * di
        return b, f, f
    if name == "gemm_f2_two_paths":  # the two-path layer's F2 (the paths' ranks add up to r)
        return kernel_work("gemm_f2_al_sut", w)
    if name == "gemm_b2_two_paths":  # the two-path layer's B2
        return kernel_work("gemm_b2_dbl_svt", w)
    if name == "gemm_sign_grads":    # read dy, a, x, db; write G_U, G_V (partials of token ranges are extra)
        b, f = M * (do + di + 2 * r) * f32 + (do + di) * r * f32, 2.0 * M * r * (do + di)
        return b, f, f
    if name == "sign_grads_reduce":  # the token ranges' partial G_U, G_V summed in order
        return 0.0, 0.0, 0.0        # (no algorithmic bytes: the method has no token ranges)
    if name == "colsum_dy_c":        # read dy and c
        return 2.0 * M * do * f32, 2.0 * M * do, 2.0 * M * do
    if name == "transpose_bits":     # one bitmap in, its transpose out (average of U and V)
        return 2 * r * (di + do) / 2 / 8, 0.0, 0.0
    if name == "colsum_finish":      # read the column partials of dh, dl, dg
        mt = -(-M // 64)  # every producer uses 64-token tiles; the fused dh launch one per rank tile
        cols = 0 if r not in (128, 256, 512) else (128 if r == 128 or mt * (r // 256) <= 128 else 256)
        rows_h = mt * (r // cols) if (not keep_c and cols) else mt
        return (rows_h * do + mt * (r + di)) * f32, 0.0, 0.0
    if name == "expand_signs":       # per launch: one bitmap in, its f16 plane and transposed plane out
        rows = (di + do) / 2         # (average of U and V)
        return rows * (r / 8 + 2 * r * 2), 0.0, 0.0
    return 0.0, 0.0, 0.0


def _code_only(text: str) -> str:
    """C/C++ source without its comments and blank space, so that editing a
    comment leaves the digest of the code as it was."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """sha256 (first 16 hex digits) of the HIP library's code (comments and
    layout left out): a profile summary records the digest of the kernels it
    measured."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "binary_rank_linear_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def note(msg: str):
    print(f"# {msg}", file=sys.stderr, flush=True)


class Layer:
    """One layer's seeded inputs, resident on the GPU, and its fwd/bwd calls
    through the C ABI (the step the benchmark times)."""

    def __init__(self, w: synth.Workload, dev, keep_c: bool):
        import torch

        import binary_rank_linear_amd as blr
        self.w, self.keep_c = w, keep_c
        note(f"workload {w.name}: generating inputs")
        self.d = synth.inputs(w)
        t = {}
        for k, v in self.d.items():
            if v.dtype == np.uint32:
                v = v.view(np.int32)
            t[k] = torch.from_numpy(v).to(dev)
        self.t = t
        M, di, do, r = w.M, w.d_in, w.d_out, w.r
        f = dict(dtype=torch.float32, device=dev)
        self.y = torch.empty((M, do), **f)
        self.ta = torch.empty((M, r), **f)
        self.tc = torch.empty((M, do), **f) if keep_c else None
        self.dx = torch.empty((M, di), **f)
        self.dh, self.dl, self.dg = torch.zeros(do, **f), torch.zeros(r, **f), torch.zeros(di, **f)
        self.ws = blr.workspace(M, di, do, r, dev)
        self.blr = blr

    def fwd(self):
        t = self.t
        self.blr.blr_forward(t["x"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], y=self.y, tape_a=self.ta,
                             tape_c=self.tc, ws=self.ws)

    def bwd(self):
        t = self.t
        self.blr.blr_backward(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], self.ta, self.tc,
                              self.w.gscale, dh=self.dh, dl=self.dl, dg=self.dg, dx=self.dx, ws=self.ws)

    def step(self):
        self.fwd()
        self.bwd()


def timed(fn, n: int) -> float:
    """Mean ms per call of fn over n calls, with events on the current stream
    (the stream the library launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def kernel_profile(blr, fn, steps: int) -> dict:
    """Per-kernel launch counts and total ms over `steps` calls of fn, from the
    HIP events the library records around each of its launches."""
    import torch
    blr.blr_profile_enable(steps * 16)
    blr.blr_profile_reset()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    prof = blr.blr_profile_read()
    blr.blr_profile_enable(0)
    return prof


def kernel_table(prof: dict, w: synth.Workload, steps: int, keep_c: bool) -> dict:
    out = {}
    for name, (count, tot_ms) in prof.items():
        avg_us = 1000.0 * tot_ms / count
        nbytes, flops, xflops = kernel_work(name, w, keep_c)
        e = {"launches_per_step": count / steps, "avg_us": round(avg_us, 3),
             "gbs": round(nbytes / (avg_us * 1e-6) / 1e9, 1) if nbytes else None,
             "tflops": round(flops / (avg_us * 1e-6) / 1e12, 1) if flops else None}
        if xflops != flops:
            e["tflops_executed"] = round(xflops / (avg_us * 1e-6) / 1e12, 1)
        out[name] = e
    return out


def roofline(prof: dict, w: synth.Workload, keep_c: bool, traffic_key: str | None, label: str = "") -> dict:
    """The dominant kernel (most time per step): its algorithmic bytes or
    flops per launch over its mean launch time, against the bound its
    intensity selects (the ridge of the published peaks)."""
    dom = max(prof, key=lambda k: prof[k][1])
    nbytes, flops, xflops = kernel_work(dom, w, keep_c)
    avg_s = prof[dom][1] / prof[dom][0] / 1000.0
    if flops and flops / nbytes > RIDGE:
        roof = {"bound": "mfma", "achieved": round(flops / avg_s / 1e12, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(traffic_key, dom) if traffic_key else None
    roof["kernel"] = dom + label
    roof["avg_us"] = round(avg_s * 1e6, 3)
    roof["algorithmic_bytes"] = int(nbytes)
    roof["flops"] = flops
    if xflops != flops:
        roof["flops_executed"] = xflops
        roof["tflops_executed"] = round(xflops / avg_s / 1e12, 2)
    return roof


def cpu_baseline(layers: list, target_s: float) -> dict:
    """The f64 oracle, as it stands, on the first tokens of the same inputs
    (every layer of the step for the MLP pair): a short calibration run, then
    a sample sized to about target_s. The oracle's cost is linear in the
    token count, so tokens/s of the sample is that of the whole workload."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        for L in layers:
            d = L.d
            oracle.forward(d["x"][:n], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"], tape=False)
            oracle.backward(d["x"][:n], d["dy"][:n], d["bits_u"], d["bits_v"], d["h"], d["l"], d["g"])
        return time.perf_counter() - t0

    M = layers[0].w.M
    n = min(M, 64)
    dt = run(n)
    # a small run's time is mostly the oracle's fixed per-call work (the
    # sign decode), so scale the sample up in a few rounds
    for _ in range(3):
        if dt >= 0.4 * target_s or n >= M:
            break
        n = int(min(M, max(n + 64, n * target_s / max(dt, 1e-3))))
        n = max(64, (n // 64) * 64) if n < M else M
        dt = run(n)
    reps = 1
    if n == M and dt < 0.4 * target_s:
        # the whole workload is the sample: repeat it for a steadier figure
        reps = max(1, int(target_s / max(dt, 1e-3)))
        dt = sum(run(n) for _ in range(reps)) / reps
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} of {M} tokens of the same workload, fwd+bwd of every layer in f64, "
                      f"{dt:.2f} s per pass, mean of {reps} pass(es)"}


def measure(names: list[str], label: str, dev, args, cpu_s: float) -> dict:
    """Times one step (fwd + bwd of every layer in `names`) and profiles its
    kernels; returns the config's report."""
    import torch
    layers = [Layer(synth.WORKLOADS[n], dev, args.keep_c) for n in names]

    def step():
        for L in layers:
            L.step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = timed(step, args.steps)
    fwd_ms = timed(lambda: [L.fwd() for L in layers], args.steps)
    bwd_ms = timed(lambda: [L.bwd() for L in layers], args.steps)
    kernels, roofs = {}, []
    for L in layers:
        prof = kernel_profile(L.blr, L.step, args.steps)
        suffix = f"@{L.w.name}" if len(layers) > 1 else ""
        for k, v in kernel_table(prof, L.w, args.steps, args.keep_c).items():
            kernels[k + suffix] = v
        r = roofline(prof, L.w, args.keep_c, L.w.name, suffix)
        roofs.append((r["avg_us"] * prof[max(prof, key=lambda k: prof[k][1])][0], r))
    roof = max(roofs, key=lambda x: x[0])[1]
    M = layers[0].w.M
    f_metric = sum(L.w.flops_metric() for L in layers)
    f_mfma = sum(L.w.flops_mfma() for L in layers)
    rep = {
        "workload": label,
        "layers": [{"name": L.w.name, "M": L.w.M, "d_in": L.w.d_in, "d_out": L.w.d_out, "r": L.w.r,
                    "gscale": L.w.gscale} for L in layers],
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(M / (ms / 1000.0), 1),
        "tflops_metric": round(f_metric / (ms / 1000.0) / 1e12, 2),
        "pct_f16_peak_metric": round(100 * f_metric / (ms / 1000.0) / 1e12 / PEAK_F16_TFLOPS, 2),
        "tflops_mfma": round(f_mfma / (ms / 1000.0) / 1e12, 2),
        "pct_f16_peak_mfma": round(100 * f_mfma / (ms / 1000.0) / 1e12 / PEAK_F16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "kernel_sum_ms": round(sum(v["avg_us"] * v["launches_per_step"] for v in kernels.values()) / 1000.0, 5),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    note(f"{label}: {ms:.4f} ms per step, {rep['tflops_metric']} TFLOP/s (metric count)")
    if not args.no_cpu_baseline and cpu_s > 0:
        note(f"{label}: oracle CPU baseline")
        rep["cpu_baseline"] = cpu_baseline(layers, cpu_s)
    rep["_layers"] = layers
    return rep


def decode_pass(L: Layer, args) -> dict:
    """The standalone sign decode (`blr_expand_signs`, the pages' `expand`):
    each of the layer's bitmaps into its f16 plane and transposed plane, one
    launch per bitmap. Algorithmic bytes per launch: the bitmap read once and
    both planes written once (rows r / 8 + 2 rows r 2)."""
    import torch
    blr, t, w = L.blr, L.t, L.w
    jobs = [(t["bits_u"], w.d_out), (t["bits_v"], w.d_in)]
    planes = [(torch.empty((rows, w.r), dtype=torch.float16, device=b.device),
               torch.empty((w.r, rows), dtype=torch.float16, device=b.device)) for b, rows in jobs]

    def run():
        for (b, rows), (pl, plt) in zip(jobs, planes):
            blr.blr_expand_signs(b, rows, w.r, plane=pl, plane_t=plt)

    run()
    prof = kernel_profile(blr, run, args.steps)
    cnt, tot = prof["expand_signs"]
    us = 1000.0 * tot / cnt
    nbytes = kernel_work("expand_signs", w)[0]
    return {"launches": 2, "avg_us": round(us, 3), "algorithmic_bytes": int(nbytes),
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def extras(L: Layer, dev, args) -> tuple[dict | None, dict | None]:
    """Context on the headline layer (not part of its step): the sign
    gradients of blr_backward_signs, and the layer of two paths of half the
    rank each (the same MFMA work as one path) through the fused entry
    points."""
    import torch
    blr, t, w = L.blr, L.t, L.w
    M, di, do, r = w.M, w.d_in, w.d_out, w.r
    gu = torch.empty((do, r), dtype=torch.float32, device=dev)
    gv = torch.empty((di, r), dtype=torch.float32, device=dev)

    def signs():
        blr.blr_backward_signs(t["x"], t["dy"], t["bits_u"], t["bits_v"], t["h"], t["l"], t["g"], L.ta, L.tc,
                               w.gscale, dh=L.dh, dl=L.dl, dg=L.dg, dx=L.dx, grad_u=gu, grad_v=gv, ws=L.ws)

    signs()
    sprof = kernel_profile(blr, signs, args.steps)
    sign = None
    if "gemm_sign_grads" in sprof:
        cnt, tot = sprof["gemm_sign_grads"]
        s_us = 1000.0 * tot / cnt
        red_us = 1000.0 * sprof["sign_grads_reduce"][1] / cnt if "sign_grads_reduce" in sprof else 0.0
        sb, sf, _ = kernel_work("gemm_sign_grads", w)
        tot_us = s_us + red_us
        sign = {"avg_us": round(s_us, 3), "reduce_us": round(red_us, 3), "total_us": round(tot_us, 3),
                "tflops": round(sf / (tot_us * 1e-6) / 1e12, 1),
                "frac_f16_peak": round(sf / (tot_us * 1e-6) / 1e12 / PEAK_F16_TFLOPS, 4),
                "gbs": round(sb / (tot_us * 1e-6) / 1e9, 1)}
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
                                   w.gscale, dh=dhp, dl=dlp, dg=dgp, dx=L.dx, ws=wsp)

        for _ in range(max(args.warmup, 1)):
            step_p()
        ms_p = timed(step_p, args.steps)
        fl = 6.0 * M * P * rp * (di + do)
        multi = {"paths": P, "rank_per_path": rp, "ms_per_step": round(ms_p, 5),
                 "tokens_per_s": round(M / (ms_p / 1000.0), 1), "tflops_metric": round(fl / (ms_p / 1000.0) / 1e12, 2)}
    return sign, multi


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=synth.HEADLINE, choices=sorted(synth.WORKLOADS) + [PAIR_NAME],
                    help="the workload of the top-level line (default: the headline layer)")
    ap.add_argument("--configs", default="all", choices=("all", "none"),
                    help="also measure every other workload under 'configs' (default) or only --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the sign-gradient and two-path context")
    ap.add_argument("--keep-c", action="store_true",
                    help="store the f32 c tape in the forward (the page's layout) instead of recomputing c")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before the run, copy a buffer of this many MiB three times with torch (a plain copy "
                         "kernel of known traffic, for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer's data-parallel split and its "
              "gradient all-reduce are not implemented here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import binary_rank_linear_amd as blr

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

    def names_of(label):
        return list(PAIR) if label == PAIR_NAME else [label]

    head = measure(names_of(args.workload), args.workload, dev, args, 10.0)
    sign = multi = decode = None
    if not args.no_extras and args.workload in synth.WORKLOADS:
        sign, multi = extras(head["_layers"][0], dev, args)
        decode = decode_pass(head["_layers"][0], args)
    del head["_layers"]
    torch.cuda.empty_cache()

    configs = {}
    if args.configs == "all":
        order = ["tiny_128x256x256_r128", "windows_2048x2048x2048_r256", synth.HEADLINE, PAIR_NAME,
                 "ragged_30000x5120x17408_r2048"]
        for label in order:
            if label == args.workload:
                continue
            rep = measure(names_of(label), label, dev, args, 3.0)
            del rep["_layers"]
            torch.cuda.empty_cache()
            configs[label] = rep

    hw = synth.WORKLOADS[names_of(args.workload)[0]]
    out = {
        "metric": "blr fwd+bwd tokens/s and TFLOP/s (% of f16 MFMA peak) at d=4096, r=512",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": hw.M, "d_in": hw.d_in, "d_out": hw.d_out, "r": hw.r,
                   "gscale": hw.gscale, "accumulate": "f32", "paths": 1,
                   "c_tape": "f32" if args.keep_c else "recomputed"},
    }
    for k in ("tflops_metric", "pct_f16_peak_metric", "tflops_mfma", "pct_f16_peak_mfma", "fwd_ms", "bwd_ms",
              "kernel_sum_ms", "kernels", "roofline"):
        out[k] = head[k]
    out["sign_grads"] = sign
    out["multi_path"] = multi
    out["decode_pass"] = decode
    out["configs"] = configs
    out["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
