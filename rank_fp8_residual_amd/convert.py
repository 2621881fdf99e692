"""Decomposition of a dense weight into the LiteLinear factors.

LiteLinear.from_dense (LiteLinear README, *Usage*, "From a dense nn.Linear")
builds the rank-r pair by an SVD of the dense weight and keeps the rest as an
e4m3fn residual with a per-tensor scale (*Features*: W ~ A.B + Q_fp8).  Here:

    W = U diag(S) V^T (torch.linalg.svd on the weight's device)
    A = U[:, :r] diag(sqrt(S[:r]))      bf16 [out, r]
    B = diag(sqrt(S[:r])) V^T[:r]       bf16 [r, in]
    Q, scale = residual_quantize(W - A B)   (the library's HIP kernels)

The pages leave the split of the singular values between A and B open; the
square root on each side is the plainest one (it balances the two factors'
magnitudes).  The SVD is a library routine; the residual and its
quantisation run in this library's kernels on the bf16 A and B actually
stored, so A B + scale dec(Q) is the weight the forward applies.
"""
from __future__ import annotations

import torch

from .litelinear import Handle, default_handle


def from_dense(W: torch.Tensor, rank: int, handle: Handle | None = None) -> dict:
    """Factors of a dense bf16 weight W [out, in] on a GPU.

    Returns {"A", "B", "Q", "scale"}: A bf16 [out, rank], B bf16 [rank, in],
    Q uint8 e4m3fn codes [out, in], scale a float32 tensor [1] on the device
    (the forward's `scale`, the README's Q_scale_inv).  rank must be a
    multiple of 8 (0 keeps everything in the residual)."""
    if W.dim() != 2 or W.dtype != torch.bfloat16 or W.device.type != "cuda":
        raise ValueError("W must be a 2-D bf16 tensor on a GPU")
    out_features, in_features = W.shape
    if rank < 0 or rank % 8 != 0 or rank > min(out_features, in_features):
        raise ValueError("rank must be a multiple of 8 and at most min(out, in)")
    h = handle or default_handle(W.device.index)
    if rank == 0:
        Q, scale = h.residual_quantize(W.contiguous(), None, None)
        return {"A": None, "B": None, "Q": Q, "scale": scale}
    U, S, Vh = torch.linalg.svd(W.float(), full_matrices=False)
    root = S[:rank].sqrt()
    A = (U[:, :rank] * root).to(torch.bfloat16).contiguous()
    B = (root[:, None] * Vh[:rank]).to(torch.bfloat16).contiguous()
    Q, scale = h.residual_quantize(W.contiguous(), A, B)
    return {"A": A, "B": B, "Q": Q, "scale": scale}
