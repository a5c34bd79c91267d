"""GPU parity of the whole DoRA linear layer (dora_linear) and of the
single-pass layer output (dora_layer_output) against the fp64 oracle.

dora_layer_output: within 1 ulp of the storage type of the oracle's
base + delta, plus the fp32 roundings of (g-1) base, the fused multiply-add
and the sum, each bounded by 2^-24 times the magnitude of its terms (y can
cancel toward zero, the terms cannot).

dora_linear: the two projections are library GEMMs whose bf16 outputs are
rounded, so the bound is derived from each rounding on the path, per
element, with u the unit of the storage type (1 ulp = 2u relative) and
e32 = 2^-24:
    base   : ulp(base) + d_in e32 (|x| |W|^T)
    u=xA^T : ulp(u) + d_in e32 (|x| |A|^T)
    lora   : ulp(lora) + err(u) |B|^T + r e32 (|u| |B|^T)
    y      : ulp(y) + |g| (err(base) + |s| err(lora))
             + (1e-5 + 4 e32) |g| (|base| + |s| |lora|)
where 1e-5 is the row norm's relative bound (so g's) and 4 e32 covers the
fp32 compose arithmetic.
"""

import numpy as np
import pytest
import torch

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I
from dora_weight_norm_amd.layer import dora_linear
from oracle import dora_oracle as O

from gpu_helpers import bf16_ulp, dev, f16_ulp, magnitude, say, ulp32

pytestmark = pytest.mark.gpu

E32 = 2.0 ** -24
EPS = 1e-6


def _ulp(x, dtype):
    return {"bf16": bf16_ulp, "f16": f16_ulp, "f32": ulp32}[dtype](x)


@pytest.mark.parametrize("T,d_out,dtype,s", [(64, 1000, "bf16", 0.5), (129, 250, "f32", 0.75),
                                             (33, 520, "bf16", 16.0 / 384 ** 0.5), (64, 1000, "f16", 0.5)])
def test_layer_output_matches_oracle(T, d_out, dtype, s):
    base, lora, g = I.compose_inputs(T, d_out, dtype, 41)
    y = bnd.dora_layer_output(dev(base, dtype), dev(lora, dtype), torch.from_numpy(g).cuda(), s)
    ref = O.layer_output(base, lora, g, s)
    got = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    # the storage rounding of y, plus the fp32 roundings of (g-1) base, the
    # fma and the sum, which scale with the terms (y may cancel toward 0)
    b64, l64, g64 = base.astype(np.float64), lora.astype(np.float64), g.astype(np.float64)[None, :]
    terms = np.abs(b64) + np.abs(g64 - 1) * np.abs(b64) + np.abs(g64) * abs(s) * np.abs(l64)
    tol = _ulp(ref, dtype) + 3 * E32 * terms
    assert np.all(err <= tol), f"worst {np.max(err / tol):.2f} of the bound"
    # in place over base, as dora_linear calls it
    bt = dev(base, dtype)
    y2 = bnd.dora_layer_output(bt, dev(lora, dtype), torch.from_numpy(g).cuda(), s, y=bt)
    assert torch.equal(y2, y)


CASES = [
    # (name, T, d_out, d_in, r, dtype, s, seed, leading shape)
    ("bf16_ragged", 64, 300, 1000, 40, "bf16", 0.5, 50, None),
    ("f32_tiny_workload", 64, 256, 256, 8, "f32", 2.0, 0, None),
    ("bf16_r384_batched", 96, 512, 2048, 384, "bf16", 0.5, 51, (2, 48)),
    ("bf16_rslora", 40, 384, 1536, 64, "bf16", 16.0 / 64 ** 0.5, 52, None),
    ("f16_r384", 64, 512, 2048, 384, "f16", 0.5, 53, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dora_linear_matches_oracle(case):
    name, T, d_out, d_in, r, dtype, s, seed, lead = case
    say(f"[linear] {name} T={T} d_out={d_out} d_in={d_in} r={r} {dtype} s={s:.4f}")
    W, A, B = I.norm_inputs(d_out, d_in, r, dtype, seed)
    x = I.activations(T, d_in, dtype, seed)
    m = magnitude(O.dense_row_norm(W, A, B, s), seed)
    xt = dev(x, dtype)
    if lead is not None:
        xt = xt.view(*lead, d_in)
    y = dora_linear(xt, dev(W, dtype), dev(A, dtype), dev(B, dtype), torch.from_numpy(m).cuda(), s, eps=EPS)
    torch.cuda.synchronize()
    assert y.shape == (*(lead or (T,)), d_out) and y.dtype == xt.dtype
    got = y.reshape(T, d_out).float().cpu().numpy().astype(np.float64)
    ref = O.dora_linear(x, W, A, B, m, s, EPS)

    xd, Wd, Ad, Bd = (v.astype(np.float64) for v in (x, W, A, B))
    base, u = xd @ Wd.T, xd @ Ad.T
    lora = u @ Bd.T
    g = np.abs(O.magnitude_scale(m, O.dense_row_norm(W, A, B, s), EPS))[None, :]
    e_base = _ulp(base, dtype) + d_in * E32 * (np.abs(xd) @ np.abs(Wd).T)
    e_u = _ulp(u, dtype) + d_in * E32 * (np.abs(xd) @ np.abs(Ad).T)
    e_lora = _ulp(lora, dtype) + e_u @ np.abs(Bd).T + r * E32 * (np.abs(u) @ np.abs(Bd).T)
    mag = np.abs(base) + abs(s) * np.abs(lora)
    tol = _ulp(ref, dtype) + g * (e_base + abs(s) * e_lora) + (1e-5 + 4 * E32) * g * mag
    err = np.abs(got - ref)
    worst = float(np.max(err / tol))
    say(f"    worst {worst:.3f} of the bound; max |err| {np.max(err):.3e}")
    assert worst <= 1.0


def test_dora_linear_rejects_mismatched_shapes():
    W = torch.zeros(8, 16, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(8, 4, dtype=torch.bfloat16, device="cuda")
    m = torch.ones(8, device="cuda")
    with pytest.raises(ValueError):
        dora_linear(torch.zeros(3, 15, dtype=torch.bfloat16, device="cuda"), W, A, B, m, 0.5)
    with pytest.raises(ValueError):
        dora_linear(torch.zeros(3, 16, dtype=torch.float32, device="cuda"), W, A, B, m, 0.5)
