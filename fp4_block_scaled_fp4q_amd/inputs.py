"""Seeded synthetic inputs for the FP4 linear workloads.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the quantization or GEMM arithmetic, and it is the one piece
that both the HIP path's tests/benchmark and the CPU oracle consume.

Value structure follows the workloads of "UE5M3 FP4 Block Scaling for Stable
Language Model Pretraining" (§1, §7: an 8B-class model's linears with
outlier-heavy activations and gradients spanning many decades; the training
data and checkpoints themselves are not available, so these stand in):

* activations: 0.5 * Student-t(3), with round(1% of columns) chosen at random
  and scaled by 50 (outlier channels);
* weights: N(0, 0.02^2) (standard deviation 0.02);
* upstream gradients: magnitude 10**U(-8, -2), fair random sign;
* the tiny case: N(0, 1) activations, N(0, 0.02^2) weights, kept in fp32.

Every tensor is drawn in float64 by numpy's default_rng in row chunks of
``CHUNK_ROWS`` rows (so the stream does not depend on available memory), cast
to float32, and for bf16 workloads rounded to bfloat16 by torch (RNE).
Held-amax companions are drawn from an independent generator (seed 1) with
the same outlier column set.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK_ROWS = 1024


def _chunked(rng: np.random.Generator, rows: int, cols: int, draw) -> np.ndarray:
    out = np.empty((rows, cols), np.float32)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = draw(rng, (r1 - r0, cols))
    return out


def outlier_columns(rng: np.random.Generator, cols: int, frac: float = 0.01) -> np.ndarray:
    n = int(round(frac * cols))
    return np.sort(rng.choice(cols, size=n, replace=False))


def activation(rng: np.random.Generator, rows: int, cols: int, outliers: np.ndarray,
               nu: float = 3.0, scale: float = 0.5, boost: float = 50.0) -> np.ndarray:
    x = _chunked(rng, rows, cols, lambda g, s: scale * g.standard_t(nu, size=s))
    if len(outliers):
        x[:, outliers] *= np.float32(boost)
    return x


def gaussian(rng: np.random.Generator, rows: int, cols: int, std: float) -> np.ndarray:
    return _chunked(rng, rows, cols, lambda g, s: std * g.standard_normal(size=s))


def loguniform_grad(rng: np.random.Generator, rows: int, cols: int,
                    lo_exp: float = -8.0, hi_exp: float = -2.0) -> np.ndarray:
    def draw(g, s):
        mag = 10.0 ** g.uniform(lo_exp, hi_exp, size=s)
        sign = np.where(g.integers(0, 2, size=s) == 0, -1.0, 1.0)
        return mag * sign
    return _chunked(rng, rows, cols, draw)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bfloat16 bit patterns as uint16 (the oracle's bf16 input form)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Tensor:
    """One workload tensor on the host: the storage-dtype torch tensor plus
    the array form the oracle reads (float32, or uint16 bfloat16 bits)."""
    name: str
    t: torch.Tensor
    held_from: torch.Tensor | None = None  # same-distribution companion for a held amax

    @property
    def oracle_view(self) -> np.ndarray:
        return self.t.numpy() if self.t.dtype == torch.float32 else bf16_bits(self.t)

    @property
    def held_oracle_view(self) -> np.ndarray:
        h = self.held_from
        return h.numpy() if h.dtype == torch.float32 else bf16_bits(h)


@dataclass
class Workload:
    name: str
    dims: dict
    tensors: dict = field(default_factory=dict)


def make(name: str, scale_rows: int | None = None, with_held: bool = True) -> Workload:
    """Build one named workload.

    ``scale_rows`` (optional) replaces the token count M, keeping the other
    sizes and the distributions; the parity tests use it for oracle-sized
    versions of the large shapes.
    """
    if name == "tiny_fwd":
        M, N, K = 64, 128, 256
        if scale_rows:
            M = scale_rows
        rng = np.random.default_rng(0)
        X = rng.standard_normal((M, K)).astype(np.float32)
        W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
        wl = Workload(name, dict(M=M, N=N, K=K))
        wl.tensors["X"] = Tensor("X", torch.from_numpy(X))
        wl.tensors["W"] = Tensor("W", torch.from_numpy(W))
        return wl

    shapes = {
        "quantize": dict(M=8192, K=4096),
        "linear_fwd": dict(M=8192, N=4096, K=4096),
        "linear_bwd": dict(M=8192, N=4096, K=4096),
        "ffn_up_step": dict(M=16384, N=14336, K=4096),
    }
    if name not in shapes:
        raise KeyError(name)
    if name == "ffn_up_step":
        with_held = False  # a refresh step: every operand's amax is sampled from itself
    dims = dict(shapes[name])
    if scale_rows:
        dims["M"] = scale_rows
    M, K = dims["M"], dims["K"]
    N = dims.get("N")
    rng = np.random.default_rng(0)
    rng_held = np.random.default_rng(1)
    wl = Workload(name, dims)

    cols = outlier_columns(rng, K)
    X = activation(rng, M, K, cols)
    Xh = activation(rng_held, M, K, cols) if with_held else None
    wl.tensors["X"] = Tensor("X", to_bf16(X), to_bf16(Xh) if Xh is not None else None)
    del X, Xh
    if name == "quantize":
        return wl
    W = gaussian(rng, N, K, 0.02)
    Wh = gaussian(rng_held, N, K, 0.02) if with_held else None
    wl.tensors["W"] = Tensor("W", to_bf16(W), to_bf16(Wh) if Wh is not None else None)
    del W, Wh
    if name == "linear_fwd":
        return wl
    dY = loguniform_grad(rng, M, N)
    dYh = loguniform_grad(rng_held, M, N) if with_held else None
    wl.tensors["dY"] = Tensor("dY", to_bf16(dY), to_bf16(dYh) if dYh is not None else None)
    return wl
