"""Seeded synthetic inputs for the fused LiteLinear forward.

This module only draws random tensors in the shapes, dtypes and value
distributions of the workloads; it holds none of the forward's arithmetic
(no e4m3 decode, no products, no bias add).  Both the HIP path and the CPU
oracle are fed from it, and neither depends on the other.

Tensor roles follow the LiteLinear README (page "moonmath-ai/LiteLinear",
Intro equation and the Features list): A is bf16 [out, r], B is bf16 [r, in]
(the same layout as ``SVDLinearLayer`` on the tt_compressor page), Q holds
OCP e4m3fn codes [out, in] in nn.Linear weight layout, ``scale`` is the
per-tensor dequantisation multiplier (the state key ``Q_scale_inv``), bias is
bf16 [out] and x is bf16 [M, in].

Recipe (the same for every workload, seed 0 unless stated):
  * one numpy ``PCG64`` generator; draws in this order: x, outlier channel
    indices (DiT only), A, B, R, bias;
  * draws are float32 standard normals scaled by the stated sigma, then
    rounded to bf16 with round-to-nearest-even (torch's cast);
  * x ~ N(0, 1); in the DiT workloads round(0.01 * in) input channels,
    chosen without replacement, are multiplied by 20 before the rounding;
  * A ~ N(0, 1/r), B ~ N(0, 1/in);
  * R ~ N(0, 0.02^2) in float32; scale = float32(max|R| / 448);
    Q = e4m3fn(clamp(R / scale, -448, 448)) with round-to-nearest-even.
    The clamp is needed because torch's cast does not saturate;
  * bias ~ N(0, 0.01^2).
With q_format="e4m3fnuz" the residual's codes are e4m3fnuz instead, with
scale = float32(max|R| / 240) and a clamp to +-240 (the format's largest
value, so the largest |R| always lands on the codes 0x7F / 0xFF).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

E4M3FN_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    in_features: int
    out_features: int
    rank: int
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    x_sigma: float = 1.0
    resid_sigma: float = 0.02
    bias_sigma: float = 0.01

    @property
    def flops(self) -> int:
        """Algorithmic flops of one forward: the three products, counted once."""
        M, K, N, r = self.M, self.in_features, self.out_features, self.rank
        return 2 * M * (K * N + r * K + r * N)

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: every input read once, y written once (bf16)."""
        M, K, N, r = self.M, self.in_features, self.out_features, self.rank
        return 2 * M * K + 2 * r * K + 2 * N * r + N * K + 2 * N + 2 * M * N


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 256, 16),
    "skinny": Workload("skinny", 16, 8192, 8192, 64),
    "llm": Workload("llm", 2048, 4096, 4096, 64),
    "dit_r32": Workload("dit_r32", 3630, 2048, 8192, 32, outlier_frac=0.01),
    "dit_r64": Workload("dit_r64", 3630, 2048, 8192, 64, outlier_frac=0.01),
    "dit_r512": Workload("dit_r512", 3630, 2048, 8192, 512, outlier_frac=0.01),
    "large": Workload("large", 16384, 4096, 16384, 512),
}


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def quantize_e4m3fn(R: torch.Tensor):
    """Per-tensor e4m3fn codes of a float32 tensor: returns (uint8 codes, scale).

    Data generation only.  The encode is torch's cast (round to nearest even);
    values are clamped to +-448 first so that nothing overflows to NaN.
    """
    R = R.to(torch.float32)
    amax = float(R.abs().max()) if R.numel() else 0.0
    scale = float(np.float32(amax / E4M3FN_MAX)) if amax > 0 else 1.0
    q = torch.clamp(R / torch.tensor(scale, dtype=torch.float32), -E4M3FN_MAX, E4M3FN_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale


E4M3FNUZ_MAX = 240.0


def quantize_e4m3fnuz(R: torch.Tensor):
    """Per-tensor e4m3fnuz codes of a float32 tensor (the residual format the
    LiteLinear README names for AMD hardware): (uint8 codes, scale), scale =
    amax / 240, so the largest magnitude lands on the code of +-240 (0x7F or
    0xFF).  Data generation only, with torch's cast (nearest even) after a
    clamp to +-240."""
    R = R.to(torch.float32)
    amax = float(R.abs().max()) if R.numel() else 0.0
    scale = float(np.float32(amax / E4M3FNUZ_MAX)) if amax > 0 else 1.0
    q = torch.clamp(R / torch.tensor(scale, dtype=torch.float32), -E4M3FNUZ_MAX, E4M3FNUZ_MAX)
    codes = q.to(torch.float8_e4m3fnuz).view(torch.uint8)
    return codes.contiguous(), scale


def make_inputs(w: Workload | str, seed: int = 0, *, M: int | None = None,
                with_bias: bool = True, q_format: str = "e4m3fn") -> dict:
    """Draw one workload's inputs as CPU tensors.

    ``M`` overrides the row count (the other draws keep their order).  Returns
    a dict with x, A, B, Q, scale, bias (None when ``with_bias`` is false) and
    the workload's shape.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    M = w.M if M is None else M
    K, N, r = w.in_features, w.out_features, w.rank
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((M, K), dtype=np.float32) * np.float32(w.x_sigma)
    n_out = int(round(w.outlier_frac * K))
    if n_out:
        cols = g.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(w.outlier_gain)
    A = g.standard_normal((N, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)) if r else np.zeros((N, 0), np.float32)
    B = g.standard_normal((r, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K)) if r else np.zeros((0, K), np.float32)
    R = g.standard_normal((N, K), dtype=np.float32) * np.float32(w.resid_sigma)
    bias = g.standard_normal((N,), dtype=np.float32) * np.float32(w.bias_sigma)
    Q, scale = (quantize_e4m3fnuz if q_format == "e4m3fnuz" else quantize_e4m3fn)(torch.from_numpy(R))
    return {
        "x": _bf16(x), "A": _bf16(A), "B": _bf16(B), "Q": Q, "scale": scale,
        "bias": _bf16(bias) if with_bias else None,
        "M": M, "in": K, "out": N, "r": r,
    }


def random_inputs(M: int, K: int, N: int, r: int, seed: int = 0, *,
                  with_bias: bool = True, x_sigma: float = 1.0, q_format: str = "e4m3fn") -> dict:
    """Inputs of an arbitrary shape drawn with the same recipe (no outliers)."""
    w = Workload(f"adhoc_{M}x{K}x{N}_r{r}", M, K, N, r, x_sigma=x_sigma)
    return make_inputs(w, seed, with_bias=with_bias, q_format=q_format)


def exact_inputs(M: int, K: int, N: int, r: int, seed: int = 0, *,
                 with_bias: bool = True) -> dict:
    """Inputs whose forward is exact in float32 under every summation order.

    x holds integers in [-4, 4]; each row of B holds at most 64 entries of
    +-1 and zeros elsewhere (so every x.B^T dot product is an integer of
    magnitude <= 256, exact in bf16); A holds {-1, 0, 1}; Q holds the codes of
    the integers -4..4 (exact in e4m3fn); scale is 1/4 and bias holds
    multiples of 1/4 in [-2, 2].  Every partial sum is then a multiple of 1/4
    far below 2^22, so any float32 accumulation order returns the exact value.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    A = g.integers(-1, 2, size=(N, r)).astype(np.float32)
    B = np.zeros((r, K), np.float32)
    nnz = min(64, K)
    for k in range(r):
        cols = g.choice(K, size=nnz, replace=False)
        B[k, cols] = g.choice(np.array([-1.0, 1.0], np.float32), size=nnz)
    qv = g.integers(-4, 5, size=(N, K)).astype(np.float32)
    bias = g.integers(-8, 9, size=(N,)).astype(np.float32) * np.float32(0.25)
    Q = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return {
        "x": _bf16(x), "A": _bf16(A), "B": _bf16(B), "Q": Q, "scale": 0.25,
        "bias": _bf16(bias) if with_bias else None,
        "M": M, "in": K, "out": N, "r": r,
    }
