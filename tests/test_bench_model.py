"""The benchmark's host-side model, without a GPU: the algorithmic bytes and
FLOPs every roofline figure divides by, the partial-row count of the finish
pass, and the source digest that decides whether a committed HBM-traffic
summary still describes the kernels."""
import os

import pytest

import bench
import synth

HEADLINE = synth.WORKLOADS["attn_proj_8192x4096x4096_r512"]
WINDOWS = synth.WORKLOADS["windows_2048x2048x2048_r256"]


def test_headline_algorithmic_bytes():
    """Each contraction's minimum HBM traffic at M = 8192, d = 4096, r = 512,
    written out from the operands it must read and write once: f32
    activations, 1-bit bitmaps, f32 per-column scales."""
    M, d, r = 8192, 4096, 512
    f1 = 4 * M * (d + r) + r * d // 8 + 4 * d          # x in, a out, S_V bits, g
    f2 = 4 * M * (r + d) + d * r // 8 + 4 * (r + d)    # a in, y out, S_U bits, l and h
    b1dh = 4 * M * (d + 2 * r) + 2 * r * d // 8 + 4 * d + 4 * r  # dy, a in, db out, S_U bits twice, h, l
    b2 = 4 * M * (r + 2 * d) + d * r // 8 + 4 * (r + d)  # db, x in, dx out, S_V bits, l, g
    for name, want in [("gemm_f1_xg_sv", f1), ("gemm_f2_al_sut", f2), ("gemm_b1_dh_fused", b1dh),
                       ("gemm_b2_dbl_svt", b2)]:
        assert bench.kernel_work(name, HEADLINE)[0] == want, name
    assert b1dh == 168314880  # the figure the headline roofline divides by


def test_fused_launch_counts_the_method_work_only():
    """The fused B1 + dh launch is credited with B1's contraction and the two
    column sums; the recomputed c (the pages read it from the tape) is
    executed work only."""
    M, d, r = 8192, 4096, 512
    _, flops, executed = bench.kernel_work("gemm_b1_dh_fused", HEADLINE)
    assert flops == 2.0 * M * r * d + 2.0 * M * r + 2.0 * M * d
    assert executed - flops == 2.0 * M * r * d
    # the metric's count per step: 6 M r (d_in + d_out) = 206.2 GFLOP
    assert 6 * M * r * (d + d) == 206158430208


@pytest.mark.parametrize("w,rows_h", [(HEADLINE, 256), (WINDOWS, 64)])
def test_finish_pass_rows(w, rows_h):
    """The fused launch writes one dh partial row per (rank tile, 64-token
    tile): 256-rank tiles at the attention projection (128 token tiles x 2),
    128-rank tiles on the 2048-token layer (32 token tiles, too few for
    256-rank tiles: 32 x 2)."""
    mt = -(-w.M // 64)
    want = (rows_h * w.d_out + mt * (w.r + w.d_in)) * 4
    assert bench.kernel_work("colsum_finish", w)[0] == want


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {\n    // doubles x\n    return 2 * x; /* the\n result */\n}\n"
    b = "int f(int x) { return 2 * x;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(b.replace("2 * x", "3 * x"))


def test_measured_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    """A traffic summary is used only while its recorded digest matches the
    kernel sources; editing a comment keeps it, editing code drops it."""
    csrc = tmp_path / "binary_rank_linear_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "k.hip"
    src.write_text("__global__ void k(float *p) { p[0] = 1.0f; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest()
    (tmp_path / "profiles" / "hbm_traffic_wl.md").write_text(
        f"# summary\n\nsource_digest: {digest}\ntraffic_bytes gemm_x: 1234\n")
    assert bench.measured_traffic("wl", "gemm_x") == 1234
    assert bench.measured_traffic("wl", "gemm_y") is None
    assert bench.measured_traffic("other", "gemm_x") is None
    src.write_text("// a comment\n__global__ void k(float *p) {\n  p[0] = 1.0f;\n}\n")
    assert bench.measured_traffic("wl", "gemm_x") == 1234
    src.write_text("__global__ void k(float *p) { p[0] = 2.0f; }\n")
    assert bench.measured_traffic("wl", "gemm_x") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    """The benchmark runs on one GPU; asked for more it says so and exits
    with status 2 before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
