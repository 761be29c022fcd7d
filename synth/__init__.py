"""Seeded synthetic inputs for the binary low-rank (`blr`) linear layer.

This module only draws numbers. It holds none of the layer's arithmetic:
no sign decode, no products, no reductions. The same arrays feed the f64
oracle, the HIP path, the tests and the benchmark.

Each workload is named by what it is and its sizes. Shapes follow the layer
of the cortiq-engine `train_mm.rs` page (module doc block and `Blr`): x is
[M][d_in], y and dy are [M][d_out], the sign bitmaps are [rows][ceil(r/32)]
u32 words (bit j of word w is rank 32w+j; a set bit is +1), h is [d_out],
l (the diagonal ell) is [r], g is [d_in].

Distributions: x ~ N(0,1) f32 (optionally with 1% of entries, chosen by an
iid Bernoulli(0.01) mask, scaled by 100); dy ~ N(0, sigma) with sigma the
standard deviation; h, g ~ U(0.5, 1.5); l ~ U(0, l_hi); bitmap words are
uniform random 32-bit words. Draws use numpy's PCG64 generator seeded per
tensor, in f64 where numpy draws in f64, then rounded to f32.

`gscale` is the caller's power-of-two gradient staging scale for the
workload: the largest power of two not above 1/(1.5*sigma), which keeps the
staged backward operands near unit magnitude in f16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# per-tensor seed offsets (the page's tests seed S_U 10, S_V 20, h 30, l 40,
# g 50, x 60, dy 61); 62 is the outlier mask
SEED_SU, SEED_SV, SEED_H, SEED_L, SEED_G, SEED_X, SEED_DY, SEED_MASK = 10, 20, 30, 40, 50, 60, 61, 62


def pow2_gscale(sigma: float) -> float:
    """Largest power of two not above 1/(1.5*sigma)."""
    return float(2.0 ** math.floor(math.log2(1.0 / (1.5 * sigma))))


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    d_in: int
    d_out: int
    r: int
    dy_sigma: float
    l_hi: float
    outliers: bool
    seed: int
    desc: str = ""
    gscale: float = field(default=0.0)

    def __post_init__(self):
        if self.gscale == 0.0:
            object.__setattr__(self, "gscale", pow2_gscale(self.dy_sigma))

    @property
    def words(self) -> int:
        return (self.r + 31) // 32

    def flops_metric(self) -> float:
        """FLOPs of one fwd+bwd under the headline count: 2*M*r*(d_in+d_out)
        forward and twice that backward."""
        return 6.0 * self.M * self.r * (self.d_in + self.d_out)

    def flops_mfma(self) -> float:
        """FLOPs the four rank-r contractions actually perform per fwd+bwd."""
        return 4.0 * self.M * self.r * (self.d_in + self.d_out)

    def with_tokens(self, M: int) -> "Workload":
        return Workload(self.name, M, self.d_in, self.d_out, self.r, self.dy_sigma, self.l_hi,
                        self.outliers, self.seed, self.desc, self.gscale)


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_128x256x256_r128", 128, 256, 256, 128, 1e-6, 0.1, False, 1000,
                 "tiny layer, M=128, d_in=d_out=256, r=128"),
        Workload("windows_2048x2048x2048_r256", 2048, 2048, 2048, 256, 1e-6, 0.1 * 16 / math.sqrt(256), False, 2000,
                 "4 windows x 512 tokens, d_in=d_out=2048, r=256, l ~ U(0,0.1)*16/sqrt(r)"),
        Workload("attn_proj_8192x4096x4096_r512", 8192, 4096, 4096, 512, 1e-6, 0.05, False, 3000,
                 "attention-projection shape, 8 x 1024 tokens, d_in=d_out=4096, r=512"),
        Workload("mlp_up_8192x4096x12288_r1024", 8192, 4096, 12288, 1024, 1e-7, 0.03, False, 4000,
                 "MLP up-projection, 4096 -> 12288, r=1024"),
        Workload("mlp_down_8192x12288x4096_r1024", 8192, 12288, 4096, 1024, 1e-7, 0.03, False, 4500,
                 "MLP down-projection, 12288 -> 4096, r=1024"),
        Workload("ragged_30000x5120x17408_r2048", 30000, 5120, 17408, 2048, 1e-6, 0.02, True, 5000,
                 "large layer with ragged tokens (30000, padded to 30080 inside), x with 1% outliers x100"),
    ]
}

HEADLINE = "attn_proj_8192x4096x4096_r512"
SMALL = "tiny_128x256x256_r128"


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def sign_bits(rows: int, r: int, seed: int) -> np.ndarray:
    """Uniform random bitmap words [rows][ceil(r/32)] u32."""
    w = (r + 31) // 32
    return rng(seed).integers(0, 1 << 32, size=(rows, w), dtype=np.uint32)


def uniform(n: int, lo: float, hi: float, seed: int) -> np.ndarray:
    return rng(seed).uniform(lo, hi, size=n).astype(np.float32)


def normal(shape, sigma: float, seed: int) -> np.ndarray:
    v = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        v *= np.float32(sigma)
    return v


def x_input(w: Workload, M: int | None = None) -> np.ndarray:
    M = w.M if M is None else M
    x = normal((M, w.d_in), 1.0, w.seed + SEED_X)
    if w.outliers:
        mask = rng(w.seed + SEED_MASK).random(size=(M, w.d_in)) < 0.01
        x[mask] *= np.float32(100.0)
    return x


def dy_input(w: Workload, M: int | None = None) -> np.ndarray:
    M = w.M if M is None else M
    return normal((M, w.d_out), w.dy_sigma, w.seed + SEED_DY)


def params(w: Workload) -> dict[str, np.ndarray]:
    """Sign bitmaps and the three diagonals of one path."""
    return {
        "bits_u": sign_bits(w.d_out, w.r, w.seed + SEED_SU),
        "bits_v": sign_bits(w.d_in, w.r, w.seed + SEED_SV),
        "h": uniform(w.d_out, 0.5, 1.5, w.seed + SEED_H),
        "l": uniform(w.r, 0.0, w.l_hi, w.seed + SEED_L),
        "g": uniform(w.d_in, 0.5, 1.5, w.seed + SEED_G),
    }


def inputs(w: Workload) -> dict[str, np.ndarray]:
    d = params(w)
    d["x"] = x_input(w)
    d["dy"] = dy_input(w)
    return d


def custom(M: int, d_in: int, d_out: int, r: int, seed: int, dy_sigma: float = 1e-3,
           l_hi: float = 0.1) -> dict[str, np.ndarray]:
    """Inputs of arbitrary shape (edge cases, ragged tails)."""
    w = Workload("custom", M, d_in, d_out, r, dy_sigma, l_hi, False, seed)
    d = inputs(w)
    d["gscale"] = np.float32(w.gscale)
    return d


def custom_paths(M: int, d_in: int, d_out: int, r: int, paths: int, seed: int, dy_sigma: float = 1e-3,
                 l_hi: float = 0.1) -> dict[str, np.ndarray]:
    """A layer of `paths` paths: x and dy of path 0's draw, and each path's
    bitmaps and scales from its own seed (seed + 97 p), stacked along a
    leading path axis."""
    per = [custom(M, d_in, d_out, r, seed + 97 * p, dy_sigma=dy_sigma, l_hi=l_hi) for p in range(paths)]
    d = {k: np.stack([q[k] for q in per]) for k in ("bits_u", "bits_v", "h", "l", "g")}
    d["x"], d["dy"], d["gscale"] = per[0]["x"], per[0]["dy"], per[0]["gscale"]
    return d


def exact_grid(M: int, d_in: int, d_out: int, r: int, seed: int) -> dict[str, np.ndarray]:
    """Inputs on a grid where every f16-staged forward operand is exact: x in
    (1/8)Z with |x| <= 1/2, g in {0.5, 1}, l in {0.5, 1, 2} (the page's
    sign-flip test uses this grid), h ~ U(0.02, 0.07)."""
    R = rng(seed)
    x = (R.integers(-4, 5, size=(M, d_in)) / 8.0).astype(np.float32)
    g = np.where(R.random(d_in) < 0.5, 0.5, 1.0).astype(np.float32)
    l = np.array([0.5, 1.0, 2.0], dtype=np.float32)[R.integers(0, 3, size=r)]
    h = R.uniform(0.02, 0.07, size=d_out).astype(np.float32)
    return {
        "x": x, "g": g, "l": l, "h": h,
        "bits_u": sign_bits(d_out, r, seed + 1),
        "bits_v": sign_bits(d_in, r, seed + 2),
    }
