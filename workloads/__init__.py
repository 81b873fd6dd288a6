"""Seeded synthetic layer workloads for the GPTQ-family layer-quantization path.

This module only *draws inputs*: weights W (K x N), calibration activations X (M x K), the float-stream
activations of asymmetric calibration, and the per-group token weights of output-channel groups.  It holds
none of the method's arithmetic (no Gram, no factorisation, no rounding to a weight grid), so that both the
float64 oracle and the HIP path can consume the very same bytes.

Shapes and value distributions follow the layer workloads the method pages describe:
  * calibration set of 1024 sequences x 2048 tokens, Hadamard rotation before quantisation, symmetric
    per-channel weight grids (G2PTQ digest, setup paragraph);
  * activations with lognormal per-channel energy and a few outlier channels, SiLU-gated MLP inputs for
    down projections, and zero-energy ("dead") input channels (GPTQ tutorial, section on damping and dead
    coordinates);
  * a quantised-stream X that differs from the float-stream X~ by a small relative perturbation (GPTAQ
    notes, asymmetric calibration).
No public dataset is used; every tensor is drawn from a seed.

Bulk arrays (W, X) are drawn with torch generators on the requested device; small per-channel vectors
(channel scales, outlier / dead picks, Hadamard signs) are drawn with numpy so they are identical on every
device.  bf16 tensors are produced by torch's round-to-nearest-even conversion from fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 0x67707471


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    K: int                 # input features (rows of W in the K x N layout)
    N: int                 # output channels
    M: int                 # calibration tokens
    x_dtype: str           # "f32" or "bf16"
    w_dtype: str           # "f32" or "bf16"
    w_sigma: float
    bits: int
    blocksize: int = 128
    percdamp: float = 0.01
    x_kind: str = "gauss"  # "gauss": c_k * N(0,1);  "silu": SiLU(a) * b * c_k
    scale_sigma: float = 1.0
    n_outliers: int = 0
    outlier_factor: float = 20.0
    hadamard: bool = False
    groups: int = 1        # output-channel groups, each with its own Hessian
    dead_frac: float = 0.0
    asym_noise: float = 0.0  # > 0: asymmetric calibration; X = bf16(X~ + eps), eps ~ N(0, (noise*|X~|)^2)
    cfg_id: int = 0

    def scaled(self, **kw) -> "LayerConfig":
        """Same recipe at other sizes (used for parity cases the oracle finishes in seconds)."""
        return dataclasses.replace(self, **kw)

    @property
    def torch_x_dtype(self):
        return torch.float32 if self.x_dtype == "f32" else torch.bfloat16

    @property
    def torch_w_dtype(self):
        return torch.float32 if self.w_dtype == "f32" else torch.bfloat16


# The five layer workloads.  Sizes are LLaMA-8B / 70B projection shapes.
CONFIGS = {
    "c1_512": LayerConfig("c1_512", K=512, N=512, M=2048, x_dtype="f32", w_dtype="f32", w_sigma=0.02,
                          bits=4, x_kind="gauss", scale_sigma=1.0, n_outliers=4, cfg_id=1),
    "c2_q_proj_8b": LayerConfig("c2_q_proj_8b", K=4096, N=4096, M=1024 * 2048, x_dtype="bf16",
                                w_dtype="bf16", w_sigma=0.02, bits=3, x_kind="gauss", scale_sigma=1.0,
                                n_outliers=4, hadamard=True, cfg_id=2),
    "c3_down_proj_8b_g4": LayerConfig("c3_down_proj_8b_g4", K=14336, N=4096, M=262144, x_dtype="bf16",
                                      w_dtype="bf16", w_sigma=0.015, bits=2, x_kind="silu",
                                      scale_sigma=0.5, groups=4, cfg_id=3),
    "c4_up_proj_8b_gptaq": LayerConfig("c4_up_proj_8b_gptaq", K=4096, N=14336, M=262144, x_dtype="bf16",
                                       w_dtype="bf16", w_sigma=0.02, bits=4, x_kind="gauss",
                                       scale_sigma=1.0, asym_noise=0.05, cfg_id=4),
    "c5_down_proj_70b": LayerConfig("c5_down_proj_70b", K=28672, N=8192, M=524288, x_dtype="bf16",
                                    w_dtype="bf16", w_sigma=0.01, bits=4, x_kind="silu", scale_sigma=0.5,
                                    dead_frac=0.01, cfg_id=5),
}


def _seed(cfg: LayerConfig, stream: str, seed: int) -> int:
    """A 63-bit seed for one named random stream of one workload."""
    tag = [ord(ch) for ch in stream]
    ss = np.random.SeedSequence([ROOT_SEED, cfg.cfg_id, seed] + tag)
    return int(ss.generate_state(2, dtype=np.uint32).astype(np.uint64) @ np.array([1, 1 << 31], np.uint64)) \
        & ((1 << 63) - 1)


def _torch_gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def channel_scales(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """Per-input-channel energy c_k (float64): lognormal, outliers scaled, dead channels zero."""
    rng = np.random.default_rng(_seed(cfg, "chan", seed))
    c = np.exp(rng.normal(0.0, cfg.scale_sigma, size=cfg.K))
    picks = rng.permutation(cfg.K)
    n_out = min(cfg.n_outliers, cfg.K)
    c[picks[:n_out]] *= cfg.outlier_factor
    n_dead = int(round(cfg.dead_frac * cfg.K))
    if n_dead:
        c[picks[n_out:n_out + n_dead]] = 0.0
    return c


def dead_channels(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    """Indices of the zero-energy input channels of the recipe (sorted)."""
    return np.sort(np.flatnonzero(channel_scales(cfg, seed) == 0.0))


def hadamard_signs(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(_seed(cfg, "hsign", seed))
    return rng.choice(np.array([-1.0, 1.0]), size=cfg.K)


def sylvester_hadamard(n: int, device="cpu") -> torch.Tensor:
    """+-1 Sylvester-Hadamard matrix of order n (power of two): entry (i, j) = (-1)^popcount(i & j)."""
    assert n > 0 and n & (n - 1) == 0
    idx = torch.arange(n, device=device)
    a = idx[:, None] & idx[None, :]
    par = torch.zeros_like(a)
    while bool((a != 0).any()):
        par ^= a & 1
        a = a >> 1
    return (1.0 - 2.0 * par).to(torch.float32)


def make_weights(cfg: LayerConfig, device="cpu", seed: int = 0) -> torch.Tensor:
    """W: K x N row-major, N(0, w_sigma^2) drawn in fp32 then rounded to the weight dtype."""
    g = _torch_gen(device, _seed(cfg, "W", seed))
    w = torch.randn(cfg.K, cfg.N, generator=g, device=device, dtype=torch.float32) * cfg.w_sigma
    return w.to(cfg.torch_w_dtype)


def make_group_row_weights(cfg: LayerConfig, device="cpu", seed: int = 0) -> Optional[torch.Tensor]:
    """rho: groups x M fp32, i.i.d. U(0.5, 1.5) per token and group (None without groups)."""
    if cfg.groups <= 1:
        return None
    g = _torch_gen(device, _seed(cfg, "rho", seed))
    return torch.rand(cfg.groups, cfg.M, generator=g, device=device, dtype=torch.float32) + 0.5


class ActivationSource:
    """Draws the calibration activations X (M x K) chunk by chunk into a caller-visible tensor.

    For asymmetric calibration it also draws the float stream X~ and returns X = bf16(X~ + eps).
    """

    def __init__(self, cfg: LayerConfig, device="cpu", seed: int = 0):
        self.cfg, self.device, self.seed = cfg, device, seed
        c = channel_scales(cfg, seed)
        self.c = torch.tensor(c, dtype=torch.float32, device=device)
        self.rot = None
        if cfg.hadamard:
            d = torch.tensor(hadamard_signs(cfg, seed), dtype=torch.float32, device=device)
            h = sylvester_hadamard(cfg.K, device=device)
            self.rot = (d[:, None] * h) / math.sqrt(cfg.K)

    def _chunk(self, gen: torch.Generator, rows: int):
        cfg = self.cfg
        if cfg.x_kind == "gauss":
            x = torch.randn(rows, cfg.K, generator=gen, device=self.device, dtype=torch.float32)
        elif cfg.x_kind == "silu":
            a = torch.randn(rows, cfg.K, generator=gen, device=self.device, dtype=torch.float32)
            b = torch.randn(rows, cfg.K, generator=gen, device=self.device, dtype=torch.float32)
            x = torch.nn.functional.silu(a) * b
            del a, b
        else:
            raise ValueError(cfg.x_kind)
        x.mul_(self.c)
        if self.rot is not None:
            x = x @ self.rot
        return x

    def fill(self, X: torch.Tensor, X_float: Optional[torch.Tensor] = None, chunk_rows: int = 32768):
        """Write all M rows into X (M x K, cfg x dtype) [and X~ for asymmetric calibration]."""
        cfg = self.cfg
        assert X.shape == (cfg.M, cfg.K) and X.dtype == cfg.torch_x_dtype
        gen = _torch_gen(self.device, _seed(cfg, "X", self.seed))
        ngen = _torch_gen(self.device, _seed(cfg, "eps", self.seed)) if cfg.asym_noise > 0 else None
        for r0 in range(0, cfg.M, chunk_rows):
            rows = min(chunk_rows, cfg.M - r0)
            x = self._chunk(gen, rows)
            if cfg.asym_noise > 0:
                assert X_float is not None and X_float.shape == X.shape
                xt = x.to(cfg.torch_x_dtype)
                X_float[r0:r0 + rows] = xt
                xf = xt.float()
                eps = torch.randn(rows, cfg.K, generator=ngen, device=self.device, dtype=torch.float32)
                X[r0:r0 + rows] = (xf + eps * (cfg.asym_noise * xf.abs())).to(cfg.torch_x_dtype)
            else:
                X[r0:r0 + rows] = x.to(cfg.torch_x_dtype)
            del x
        return X


def make_activations(cfg: LayerConfig, device="cpu", seed: int = 0):
    """Returns (X, X_float or None) as freshly allocated tensors on `device`."""
    X = torch.empty(cfg.M, cfg.K, dtype=cfg.torch_x_dtype, device=device)
    Xf = torch.empty_like(X) if cfg.asym_noise > 0 else None
    ActivationSource(cfg, device, seed).fill(X, Xf)
    return X, Xf


def make_layer(cfg: LayerConfig, device="cpu", seed: int = 0) -> dict:
    X, Xf = make_activations(cfg, device, seed)
    return {
        "cfg": cfg,
        "W": make_weights(cfg, device, seed),
        "X": X,
        "X_float": Xf,
        "rho": make_group_row_weights(cfg, device, seed),
    }


def random_spd(K: int, seed: int, log_spread: float = 2.0) -> np.ndarray:
    """A generic symmetric positive-definite K x K float64 matrix Q diag(lam) Q^T.

    Q is a random orthogonal matrix (QR of a Gaussian matrix) and the eigenvalues lam are lognormal with
    the given spread; used as a stand-in Hessian for the factorisation stage on its own.
    """
    rng = np.random.default_rng(seed)
    q, r = np.linalg.qr(rng.normal(size=(K, K)))
    q = q * np.sign(np.diag(r))
    lam = np.exp(rng.normal(0.0, log_spread / 2.0, size=K))
    return (q * lam) @ q.T
