"""Shared pieces of the GPU parity tests (inputs, oracle references, bounds)."""

import numpy as np
import torch

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I
from oracle import dora_oracle as O

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}
NORM_RTOL = 1e-5          # wnorm vs the fp64 oracle, relative


def say(msg: str) -> None:
    print(msg, flush=True)


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage-exact float32 values -> device tensor of the storage dtype (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DT[dtype])


def norm_case(d_out, d_in, r, dtype, seed):
    W, A, B = I.norm_inputs(d_out, d_in, r, dtype, seed)
    return W, A, B


def magnitude(wnorm_ref: np.ndarray, seed: int) -> np.ndarray:
    """m = fp32(wnorm * (1 + 0.0015 N(0,1))), from the oracle's wnorm."""
    noise = I.m_noise(wnorm_ref.shape[0], seed)
    return (wnorm_ref * (1.0 + I.G_SPREAD * noise)).astype(np.float32)


def check_norm(wnorm_gpu: np.ndarray, ref: np.ndarray, rtol: float = NORM_RTOL):
    wnorm_gpu = wnorm_gpu.astype(np.float64)
    err = np.abs(wnorm_gpu - ref)
    bad = err > rtol * np.abs(ref)
    assert not bad.any(), (
        f"{bad.sum()} of {bad.size} rows off; worst rel {np.max(err / np.maximum(np.abs(ref), 1e-300)):.3e} "
        f"at row {int(np.argmax(err / np.maximum(np.abs(ref), 1e-300)))}")
    return float(np.max(err / np.maximum(np.abs(ref), 1e-300)))


KAPPA_STRICT = 100.0      # rows up to this term-size condition number keep NORM_RTOL
TERM_RTOL = 2.0 ** -16    # ill-conditioned rows: error of wnorm^2 against the terms' size


def check_norm_conditioned(wnorm_gpu: np.ndarray, ref: np.ndarray, W, A, B, s: float):
    """NORM_RTOL on every row whose three-term evaluation is well
    conditioned, and a bound on the rest that the fp32 evaluation of the
    identity can meet.

    The kernels form wnorm^2 = ||W_j||^2 + 2s <B_j, U_j> + s^2 (B G B^T)_jj
    in fp32 (G as bf16 hi + lo for the 16-bit types, at most 2^-18 of each
    entry off). Rounding errors then scale with the size of the terms,
    T_j = ||W_j||^2 + 2|s| sum_l |B_jl U_jl| + s^2 sum_lm |B_jl| |G_lm| |B_jm|,
    not with wnorm^2: where kappa_j = T_j / wnorm_j^2 is large (W_j nearly
    cancels s (BA)_j, or G has far lower rank than r so that B G B^T
    cancels), no fp32 evaluation of the identity meets a relative bound.
    Rows with kappa_j <= KAPPA_STRICT must meet NORM_RTOL; the others must
    have |wnorm^2 - ref^2| <= TERM_RTOL * T_j (a dropped or mis-scaled term
    is off by a sizeable fraction of T_j). kappa is computed only for rows
    that miss NORM_RTOL."""
    wn = wnorm_gpu.astype(np.float64)
    rel = np.abs(wn - ref) / np.maximum(np.abs(ref), 1e-300)
    bad = np.nonzero(rel > NORM_RTOL)[0]
    if bad.size == 0:
        return float(rel.max()), 0
    W = np.asarray(W, np.float64)[bad]
    B64 = np.asarray(B, np.float64)
    Bb = B64[bad]
    A64 = np.asarray(A, np.float64)
    U = W @ A64.T
    G = A64 @ A64.T
    T = (W * W).sum(1) + 2 * abs(s) * (np.abs(Bb) * np.abs(U)).sum(1) + \
        s * s * ((np.abs(Bb) @ np.abs(G)) * np.abs(Bb)).sum(1)
    kappa = T / np.maximum(ref[bad] ** 2, 1e-300)
    assert np.all(kappa > KAPPA_STRICT), (
        f"row {int(bad[np.argmin(kappa)])} has kappa {kappa.min():.1f} and rel err {rel[bad][np.argmin(kappa)]:.3e}")
    err2 = np.abs(wn[bad] ** 2 - ref[bad] ** 2)
    assert np.all(err2 <= TERM_RTOL * T), (
        f"row {int(bad[np.argmax(err2 / T)])}: |wnorm^2 - ref^2| = {np.max(err2 / T):.3e} of the terms' size")
    return float(rel[np.setdiff1d(np.arange(ref.size), bad)].max(initial=0.0)), int(bad.size)


def check_g(g_gpu: np.ndarray, m: np.ndarray, wnorm_ref: np.ndarray, eps: float):
    g_ref = O.magnitude_scale(m, wnorm_ref, eps)
    rel = np.abs(g_gpu.astype(np.float64) - g_ref) / np.abs(g_ref)
    # wnorm's bound plus one fp32 rounding of the division
    assert np.max(rel) <= NORM_RTOL + 2.0 ** -23, np.max(rel)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(ax)[1] - 8)


def ulp32(x: np.ndarray) -> np.ndarray:
    """Spacing of binary32 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(ax)[1] - 24)


def f16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of binary16 numbers at |x| (2^-24 in the subnormal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return np.ldexp(1.0, np.frexp(ax)[1] - 11)


def storage_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """The compose bar's unit: a bf16 ulp for bf16 and fp32 storage (fp32 also
    gets its own tighter bound), an fp16 ulp for fp16 storage."""
    return f16_ulp(x) if dtype == "f16" else bf16_ulp(x)


def check_compose(out_gpu: torch.Tensor, base, lora, g, s, dtype):
    """The bar: within 1 ulp of the oracle's output (bf16 ulp for bf16 and
    fp32 storage, fp16 ulp for fp16).

    bf16, f16: |out - RNE(ref)| <= 1 ulp of the storage type.
    f32 : additionally the bound the evaluation order implies,
          fma(g, RN(s*lora), RN((g-1)*base)): half an ulp of each rounded
          operand plus one ulp of the result.
    Where the two terms nearly cancel (the output is a tiny difference of
    terms thousands of times larger), their fp32 roundings alone exceed an
    ulp of the output, so there the bar widens by those roundings,
    2^-23 (|(g-1) base| + |g s lora|); it stays 1 ulp wherever that is at
    most a sixteenth of an ulp. Returns the worst error in ulps.
    """
    ref = O.compose(base, lora, g, s)
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - O.round_to_dtype(ref, dtype))
    ub = storage_ulp(ref, dtype)
    g64 = np.asarray(g, np.float64)[None, :]
    terms = np.abs((g64 - 1.0) * np.asarray(base, np.float64)) + np.abs(g64 * s * np.asarray(lora, np.float64))
    rounding = 2.0 ** -23 * terms
    strict = rounding <= ub / 16
    assert np.all(err[strict] <= ub[strict]), f"max err {np.max(err[strict] / ub[strict]):.2f} ulp"
    assert np.all(err <= ub + rounding), f"cancelling element off by {np.max(err / (ub + rounding)):.2f}x its bound"
    if dtype == "f32":
        g2 = np.asarray(g, np.float64)[None, :]
        t = np.abs((g2 - 1.0) * base)
        sl = np.abs(s * np.asarray(lora, np.float64))
        tol = 0.5 * ulp32(t) + 0.5 * ulp32(sl) * np.abs(g2) + ulp32(np.maximum(np.abs(ref), np.abs(got)))
        e32 = np.abs(got - ref)
        assert np.all(e32 <= tol), f"fp32 bound exceeded by {np.max(e32 / tol):.2f}x"
    return float(np.max(err[strict] / ub[strict])) if strict.any() else 0.0
