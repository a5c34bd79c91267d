"""Plain fp64 CPU oracle for the DoRA factored row-norm and magnitude compose.

TEST INFRASTRUCTURE. This module is the slow, obviously-correct reference
that the HIP library (libdora) is checked against. Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The library and its Python binding never import, call or link
anything here, and nothing here imports the library.

Every number is computed in IEEE fp64 from the exact input values (bf16 and
fp32 inputs convert to fp64 without error). Matrix products use numpy's
``@`` as a library primitive; nothing is blocked, fused or reordered beyond
what the definition states, except that rows are processed in independent
row blocks to bound memory (each row's arithmetic is unchanged by that).

Pages followed (cited by title and section):

[P1] "DoRA优化技术解析：从内存瓶颈到高效实现" (cyqw.cn/news/889173):
     §1.1 (the row norm the forward pass needs), §1.2 and §1.2.1 (the
     three-term split into base, cross and Gram terms), §1.2.2 (fp32 norm,
     the clamp at 0, the decoupled magnitude division), §1.3 Table 1 (memory
     closed forms), §2.1 and §2.1.1 (the stable compose and the naive form it
     replaces), §5.1 Algorithm 1 (its chunk-size rule).
[P2] "Scaling DoRA: High-Rank Adaptation via Factored Norms and Fused
     Kernels" (alanhou.org summary of arXiv 2603.22276): "The Problem"
     (W' = m * (W + sBA) / ||W + sBA||_row) and "Factored Norm" (the
     squared-norm identity, U = W A^T, G = A A^T).
[P4] "LoRA 的工程账本" (d7kj.com): §4 and §8 (bf16 keeps 8 significant bits;
     rounding to it is round-to-nearest-even).
[P3] "Qwen LoRA 显存" (wuyublog.tech): the LoRA layouts A in R^{r x d_in},
     B in R^{d_out x r}.

Readings taken where the pages are garbled or silent (the extraction lost
most '+', '=' and '<' characters on P1):
  * The squared norm is base + 2 s cross + s^2 ba, with '+' restored as P2's
    formula shows; "s0" in Algorithm 1's notes means s == 0.
  * The chunk size rounds floor(budget / (4 d_out)) DOWN to a multiple of
    64, never below 64 and never above d_in; the last chunk may be short.
  * The compose returns the delta (g-1)*base + g*(s*lora); the layer output
    is base + delta (P1 §2.1.1 calls the naive g*(s*lora+base) - base form
    algebraically equal, which fixes this meaning).
  * g = m / max(wnorm, eps); a NaN wnorm propagates (PyTorch's clamp_min
    semantics), so the clamps below are written as comparisons.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "f32_round",
    "f16_round",
    "dense_row_norm",
    "chunk_size",
    "factored_row_norm",
    "factored_terms",
    "magnitude_scale",
    "compose",
    "compose_naive",
    "compose_f32_stable",
    "compose_f32_naive",
    "compose_backward",
    "layer_output",
    "dora_linear",
    "round_to_dtype",
    "table1_memory",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Rounding to the storage types.
# --------------------------------------------------------------------------

_BF16_SIG_BITS = 8          # 1 implicit + 7 stored mantissa bits  [P4 §4]
_BF16_MIN_EXP = -126        # same exponent range as IEEE binary32
_BF16_MAX_EXP = 127


def bf16_round(x):
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and the binary32 exponent range [P4 §4,
    §8]. For |x| in [2^(e-1), 2^e) the spacing of bf16 values is 2^(e-1-7);
    below the normal range the spacing stays 2^(-126-7). The quotient
    |x| / spacing is exact in fp64 (a power-of-two scaling), so rint() on it
    performs the round-half-to-even step exactly. Results are returned as
    fp64 holding the bf16 value.
    """
    x = _f64(x)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    ax_f = np.where(finite, ax, 0.0)
    _, e = np.frexp(ax_f)                          # ax = f * 2^e, f in [0.5, 1)
    e_eff = np.maximum(e, _BF16_MIN_EXP + 1)       # subnormal spacing is fixed
    spacing = np.ldexp(1.0, e_eff - 1 - (_BF16_SIG_BITS - 1))
    q = np.rint(ax_f / spacing) * spacing
    q = np.where(q >= np.ldexp(1.0, _BF16_MAX_EXP + 1), np.inf, q)
    out = np.copysign(q, x)
    return np.where(finite, out, x)


def f32_round(x):
    """Round fp64 values once to IEEE binary32, nearest even (numpy's
    float64 -> float32 conversion, a correctly rounded library routine);
    returned as fp64. Overflow goes to +-inf, as IEEE rounding does."""
    with np.errstate(over="ignore"):
        return _f64(x).astype(np.float32).astype(np.float64)


def f16_round(x):
    """Round fp64 values once to IEEE binary16, nearest even (numpy's
    float64 -> float16 conversion, a correctly rounded library routine);
    returned as fp64. Overflow goes to +-inf, as IEEE rounding does."""
    with np.errstate(over="ignore"):
        return _f64(x).astype(np.float16).astype(np.float64)


def round_to_dtype(x, dtype: str):
    """Round once from fp64 to the output storage type ('bf16', 'f16' or 'f32')."""
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f16":
        return f16_round(x)
    if dtype == "f32":
        return f32_round(x)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# The row norm, by its definition.
# --------------------------------------------------------------------------

def dense_row_norm(W, A, B, s, row_block: int = 2048):
    """wnorm[j] = || W[j,:] + s * (B @ A)[j,:] ||_2, in fp64.

    This is the norm in DoRA's weight form W' = m * (W + sBA)/||W + sBA||_row
    [P2 "The Problem"; P1 §1.1], computed the plain way: the dense adapted
    weight W + s*B@A is formed (one row block at a time; rows are
    independent) and each row's Euclidean norm is taken.

    Shapes follow the LoRA layouts [P3; P4]: W [d_out, d_in], A [r, d_in],
    B [d_out, r].
    """
    W = _f64(W)
    A = _f64(A)
    B = _f64(B)
    d_out = W.shape[0]
    out = np.empty(d_out, dtype=np.float64)
    for j0 in range(0, d_out, row_block):
        j1 = min(d_out, j0 + row_block)
        Wp = W[j0:j1] + s * (B[j0:j1] @ A)
        out[j0:j1] = np.sqrt(np.sum(Wp * Wp, axis=1))
    return out


# --------------------------------------------------------------------------
# The factored norm, from the squared-norm identity.
# --------------------------------------------------------------------------

def chunk_size(d_out: int, d_in: int, budget_bytes: int) -> int:
    """Chunk width of the factored norm's d_in loop [P1 §5.1 Algorithm 1, step 1].

    The fp32 chunk buffer [d_out, cs] must fit the byte budget, and the
    width is aligned to 64 elements for the matrix units. Reading: round
    floor(budget / (4 d_out)) down to a multiple of 64, keep it at least 64,
    and never exceed d_in. (The identity below holds for any split of d_in,
    so the width decides memory only, never the value.)
    """
    if d_out <= 0 or d_in <= 0:
        return max(d_in, 0)
    raw = budget_bytes // (4 * d_out)
    aligned = max(64, (raw // 64) * 64)
    return min(d_in, aligned)


def factored_terms(W, A, B):
    """The three per-row terms of the squared-norm identity, in fp64.

    Expanding ||W_j + s (BA)_j||^2 gives ||W_j||^2 + 2s <W_j, (BA)_j> +
    s^2 ||(BA)_j||^2 [P2 "Factored Norm"; P1 §1.2, §1.2.1]. Each term is
    rewritten without forming BA, with U = W A^T [d_out, r] and the Gram
    matrix G = A A^T [r, r]:
      base[j]  = sum_k W[j,k]^2
      cross[j] = <W_j, B_j A> = sum_l B[j,l] U[j,l]
      ba[j]    = ||B_j A||^2 = B_j G B_j^T = sum_l (B G)[j,l] B[j,l]
    Whole matrices, one library product each. Returns (base, cross, ba, G).
    """
    W = _f64(W)
    A = _f64(A)
    B = _f64(B)
    base = np.sum(W * W, axis=1)
    U = W @ A.T
    cross = np.sum(B * U, axis=1)
    G = A @ A.T
    ba = np.sum((B @ G) * B, axis=1)
    return base, cross, ba, G


def factored_row_norm(W, A, B, s):
    """wnorm = sqrt(max(base + 2 s cross + s^2 ba, 0)) [P1 §1.2.2; P2 "Factored Norm"].

    The clamp at 0 guards the rounding of an exact cancellation. When s == 0
    the cross and Gram terms vanish and only base remains [P1 §5.1 notes].
    """
    W = _f64(W)
    if s == 0.0:
        v = np.sum(W * W, axis=1)
    else:
        base, cross, ba, _ = factored_terms(W, A, B)
        v = base + 2.0 * s * cross + s * s * ba
    v = np.where(v < 0.0, 0.0, v)
    return np.sqrt(v)


def magnitude_scale(m, wnorm, eps: float):
    """g = m / max(wnorm, eps) [P1 §1.2.2]; a NaN wnorm stays NaN."""
    m = _f64(m)
    wnorm = _f64(wnorm)
    d = np.where(wnorm < eps, eps, wnorm)
    return m / d


# --------------------------------------------------------------------------
# The magnitude compose.
# --------------------------------------------------------------------------

def compose(base, lora, g, s):
    """delta[t,j] = (g[j] - 1) * base[t,j] + g[j] * (s * lora[t,j]), in fp64.

    The stable form of the DoRA compose [P1 §2.1, §2.1.1, §5.2]: the small
    correction (g - 1) is kept explicit, s*lora is formed before the product
    with g. base and lora are [T, d_out]; g is [d_out] and scales columns.
    """
    base = _f64(base)
    lora = _f64(lora)
    g = _f64(g)[None, :]
    return (g - 1.0) * base + g * (s * lora)


def compose_backward(dy, base, lora, g, s, wnorm=None, eps=None):
    """Gradients of the compose delta with respect to base, lora, g (and m).

    The pages describe a fused backward of the compose and report its speed
    [P1 §4.2, §5.2, §6.1 Table 9] but print no formulas. Reading: the
    plainest derivative of delta = (g - 1) * base + g * (s * lora), with g a
    per-column constant for base and lora and the row norm detached (it is
    not differentiated through), so for L = sum(dy * delta):

        d_base[t,j] = (g[j] - 1) * dy[t,j]
        d_lora[t,j] = g[j] * s * dy[t,j]
        dg[j]       = sum_t dy[t,j] * (base[t,j] + s * lora[t,j])
        dm[j]       = dg[j] / max(wnorm[j], eps)      (g = m / max(wnorm, eps))

    All in fp64. Returns (d_base, d_lora, dg) or, with wnorm, (d_base,
    d_lora, dg, dm).
    """
    dy = _f64(dy)
    base = _f64(base)
    lora = _f64(lora)
    g = _f64(g)
    gc = g[None, :]
    d_base = (gc - 1.0) * dy
    d_lora = gc * (s * dy)
    dg = np.sum(dy * (base + s * lora), axis=0)
    if wnorm is None:
        return d_base, d_lora, dg
    return d_base, d_lora, dg, dg / np.where(_f64(wnorm) < eps, eps, _f64(wnorm))


def layer_output(base, lora, g, s):
    """y = base + delta, the DoRA layer's output from its two projections.

    The compose delta is what the layer adds to the base projection
    [P1 §2.1.1]; fp64.
    """
    return _f64(base) + compose(base, lora, g, s)


def dora_linear(x, W, A, B, m, s, eps):
    """The DoRA linear layer from its definition [P2 "The Problem"].

    The adapted weight is W' = m * V / max(||V||_row, eps) with the
    direction V = W + s B A, rows scaled by the magnitude m; the layer maps
    x [T, d_in] to y = x W'^T [T, d_out]. Everything in fp64 with V formed
    densely (weight space), which is independent of the activation-space
    route the library takes (x W^T and (x A^T) B^T, then the compose).
    """
    x, W, A, B, m = (_f64(v) for v in (x, W, A, B, m))
    V = W + s * (B @ A)
    wn = np.sqrt(np.sum(V * V, axis=1))
    scale = m / np.where(wn < eps, eps, wn)
    return x @ (scale[:, None] * V).T


def compose_naive(base, lora, g, s):
    """g * (s*lora + base) - base, the algebraically equal naive form [P1 §2.1.1]."""
    base = _f64(base)
    lora = _f64(lora)
    g = _f64(g)[None, :]
    return g * (s * lora + base) - base


def compose_f32_stable(base, lora, g, s):
    """The stable form evaluated in binary32, one rounding per operation.

    Inputs are rounded to binary32 on entry; then s*lora, g-1, (g-1)*base,
    g*(s*lora) and their sum are each rounded once (numpy float32
    arithmetic, no fused multiply-add). Used only to show the cancellation
    the pages describe [P1 §2.1.1]: with g near 1 this stays close to the
    fp64 result.
    """
    f = np.float32
    base = np.asarray(base, f)
    lora = np.asarray(lora, f)
    g = np.asarray(g, f)[None, :]
    sl = f(s) * lora
    return (g - f(1.0)) * base + g * sl


def compose_f32_naive(base, lora, g, s):
    """The naive form in binary32, one rounding per operation (inputs rounded
    on entry, then s*lora, + base, g*(.), - base); it loses the (g-1)
    correction near g = 1 [P1 §2.1.1]."""
    f = np.float32
    base = np.asarray(base, f)
    lora = np.asarray(lora, f)
    g = np.asarray(g, f)[None, :]
    return g * (f(s) * lora + base) - base


# --------------------------------------------------------------------------
# Memory closed forms.
# --------------------------------------------------------------------------

def table1_memory(d_out: int, d_in: int, r: int, elem_bytes: int = 4):
    """Working-memory closed forms compared in [P1 §1.3 Table 1].

    dense   : the materialised BA product, d_out x d_in elements;
    factored: U (d_out x r) plus G (r x r);
    gram    : G alone;
    chunk   : the [d_out, cs] fp32 chunk buffer at the default 256 MiB budget.
    All in bytes.
    """
    cs = chunk_size(d_out, d_in, 256 << 20)
    return {
        "dense": d_out * d_in * elem_bytes,
        "factored": (d_out * r + r * r) * elem_bytes,
        "gram": r * r * elem_bytes,
        "chunk": d_out * cs * 4,
    }
