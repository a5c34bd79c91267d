"""The whole DoRA linear layer forward on the GPU.

The adapted weight is W' = m * V / max(||V||_row, eps) with the direction
V = W + s B A ("Scaling DoRA: High-Rank Adaptation via Factored Norms and
Fused Kernels", alanhou.org, "The Problem"), and the layer maps x to
y = x W'^T. It is evaluated in activation space, so V is never formed:

    base  = x W^T                  hipBLASLt (torch.mm)
    lora  = (x A^T) B^T            hipBLASLt (torch.mm), rank r in between
    g     = m / max(||V||_row, eps)   libdora factored norm
    y     = base + delta           libdora layer output: delta = (g-1) base
                                   + g (s lora) in fp32, base added in fp32,
                                   one rounding, one pass over base and lora

("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §2.1 and §2.1.1: the
compose delta is added to the base projection.) The two projections are
plain library GEMMs; the norm and the output run in libdora's kernels, so
the function fails with the library's loader error when libdora is missing.
"""

from __future__ import annotations

import torch

from . import binding as bnd

__all__ = ["dora_linear"]


def dora_linear(x, W, A, B, m, s: float, eps: float = 1e-6, budget_bytes: int = bnd.DEFAULT_BUDGET,
                workspace=None, stream=None):
    """y = x (m * V / max(||V||_row, eps))^T with V = W + s B A.

    x [..., d_in]; W [d_out, d_in], A [r, d_in], B [d_out, r], all of one
    storage dtype (bfloat16 or float32) on the GPU; m float32 [d_out].
    Returns y [..., d_out] in the storage dtype. Runs on `stream` (default:
    the current stream); the projections use only 2-D matrix products.
    """
    bnd.load()
    if x.dim() < 2:
        raise ValueError("x must be [..., d_in]")
    if x.dtype != W.dtype or A.dtype != W.dtype or B.dtype != W.dtype:
        raise ValueError("x, W, A and B must share a dtype")
    d_in = W.shape[1]
    if x.shape[-1] != d_in or A.shape[1] != d_in or B.shape[1] != A.shape[0] or B.shape[0] != W.shape[0]:
        raise ValueError("shapes must be x [..., d_in], W [d_out, d_in], A [r, d_in], B [d_out, r]")
    lead = x.shape[:-1]
    x2 = x.reshape(-1, d_in).contiguous()
    st = torch.cuda.current_stream() if stream is None else stream
    with torch.cuda.stream(st):
        base = torch.mm(x2, W.t())
        lora = torch.mm(torch.mm(x2, A.t()), B.t())
        _, g = bnd.dora_factored_norm(W, A, B, s, budget_bytes, m=m, eps=eps, workspace=workspace, stream=st)
        y = bnd.dora_layer_output(base, lora, g, s, y=base, stream=st)   # in place over base
    return y.reshape(*lead, W.shape[0])
