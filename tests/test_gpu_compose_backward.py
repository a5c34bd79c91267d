"""GPU parity of dora_compose_backward against the fp64 oracle.

d_base and d_lora: within 1 bf16 ulp of the oracle (each is one or two fp32
roundings of an exact product, then one rounding to the storage type; for
fp32 storage also within the fp32 bound the evaluation order implies).
dg: within the recursive-summation bound of its fixed-order fp32 sum,
    |dg - dg_ref| <= (n + 2) * 2^-24 * sum_t |dy| * (|base| + |s * lora|),
n = T terms (each term is fma(dy, fma(s, lora, base), acc)). dm: that plus
one fp32 division rounding.
"""

import numpy as np
import pytest
import torch

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I
from oracle import dora_oracle as O

from gpu_helpers import dev, say, storage_ulp, ulp32

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _inputs(T, d_out, dtype, seed):
    base, lora, g = I.compose_inputs(T, d_out, dtype, seed)
    dy, _ = I.grad_inputs(T, d_out, dtype, seed)
    return dy, base, lora, g


def _check_elem(got_t, ref, dtype, what):
    got = got_t.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - O.round_to_dtype(ref, dtype))
    ub = storage_ulp(ref, dtype)
    assert np.all(err <= ub), f"{what}: max err {np.max(err / ub):.2f} ulp"
    if dtype == "f32":
        e32 = np.abs(got - ref)
        assert np.all(e32 <= 2 * ulp32(np.abs(ref))), f"{what}: fp32 bound exceeded"


def _check_dg(dg_t, dy, base, lora, s, ref_dg, rows=None):
    got = dg_t.cpu().numpy().astype(np.float64)
    T = dy.shape[0]
    mag = np.sum(np.abs(dy.astype(np.float64)) * (np.abs(base.astype(np.float64)) +
                                                  np.abs(s * lora.astype(np.float64))), axis=0)
    tol = (T + 2) * U32 * mag + 1e-30
    err = np.abs(got - ref_dg)
    assert np.all(err <= tol), f"dg: worst {np.max(err / tol):.3f} of the bound"
    return float(np.max(err / tol))


CASES = [
    ("tiny_f32_256x256_r8", 64, 256, "f32", 2.0, 0),
    ("qproj_4096x4096_r64", 4096, 4096, "bf16", 2.0, 1),
    ("kv_512x3584_r768", 8192, 512, "bf16", 0.25, 40),
    ("ragged_bf16", 37, 1001, "bf16", 0.5, 5),
    ("ragged_f32", 129, 250, "f32", 0.75, 6),
    ("one_row", 1, 8, "bf16", 2.0, 7),
    ("f16", 256, 2048, "f16", 0.5, 8),
    ("f16_ragged", 37, 1001, "f16", 0.75, 9),
    # narrow workgroups and their row lanes: 128 strips (2 lanes), 192
    # strips (1 lane), and 64 strips (4 lanes) with fewer rows than lanes
    ("lanes2_1024", 300, 1024, "bf16", 0.5, 14),
    ("tpb192_1536", 257, 1536, "bf16", 0.25, 15),
    ("lanes4_three_rows", 3, 512, "bf16", 2.0, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_compose_backward_matches_oracle(case):
    name, T, d_out, dtype, s, seed = case
    say(f"[compose-bwd] {name} T={T} d_out={d_out} {dtype} s={s}")
    dy, base, lora, g = _inputs(T, d_out, dtype, seed)
    _, wnorm = I.grad_inputs(T, d_out, dtype, seed)
    d_base, d_lora, dg, dm = bnd.dora_compose_backward(dev(dy, dtype), dev(base, dtype), dev(lora, dtype),
                                                       torch.from_numpy(g).cuda(), s,
                                                       wnorm=torch.from_numpy(wnorm).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    rb, rl, rg, rm = O.compose_backward(dy, base, lora, g, s, wnorm=wnorm, eps=1e-6)
    _check_elem(d_base, rb, dtype, "d_base")
    _check_elem(d_lora, rl, dtype, "d_lora")
    worst = _check_dg(dg, dy, base, lora, s, rg)
    # dm = dg / max(wnorm, eps): the dg bound scaled, plus one division rounding
    got_dm = dm.cpu().numpy().astype(np.float64)
    got_dg = dg.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_dm, O.magnitude_scale(got_dg, wnorm, 1e-6) * 1.0, rtol=2 * U32, atol=0)
    say(f"    dg worst {worst:.3f} of its bound")


def test_compose_backward_headline_sampled_rows():
    w = I.HEADLINE
    T, d_out, s = w.T, w.d_out, w.s
    say(f"[compose-bwd-full] T={T} d_out={d_out}")
    dy, base, lora, g = _inputs(T, d_out, w.dtype, w.seed)
    d_base, d_lora, dg, _ = bnd.dora_compose_backward(dev(dy, "bf16"), dev(base, "bf16"), dev(lora, "bf16"),
                                                      torch.from_numpy(g).cuda(), s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 61, replace=False)]))
    rows_t = torch.from_numpy(rows).cuda()
    rb, rl, _ = O.compose_backward(dy[rows], base[rows], lora[rows], g, s)
    _check_elem(d_base[rows_t], rb, "bf16", "d_base")
    _check_elem(d_lora[rows_t], rl, "bf16", "d_lora")
    # dg over every row, the oracle summed in row blocks
    ref = np.zeros(d_out)
    for t0 in range(0, T, 1024):
        ref += O.compose_backward(dy[t0:t0 + 1024], base[t0:t0 + 1024], lora[t0:t0 + 1024], g, s)[2]
    worst = _check_dg(dg, dy, base, lora, s, ref)
    say(f"    dg worst {worst:.3f} of its bound")


def test_compose_backward_frozen_magnitude_reads_no_base_or_lora():
    T, d_out, s = 64, 1024, 0.5
    dy, base, lora, g = _inputs(T, d_out, "bf16", 11)
    d_base, d_lora, dg, dm = bnd.dora_compose_backward(dev(dy, "bf16"), None, None, torch.from_numpy(g).cuda(), s,
                                                       need_dg=False)
    assert dg is None and dm is None
    rb, rl, _ = O.compose_backward(dy, base, lora, g, s)
    _check_elem(d_base, rb, "bf16", "d_base")
    _check_elem(d_lora, rl, "bf16", "d_lora")


def test_compose_backward_closed_forms_and_determinism():
    T, d_out, s = 48, 4096, 0.5
    dy, base, lora, g = _inputs(T, d_out, "bf16", 12)
    ones = torch.ones(d_out, dtype=torch.float32, device="cuda")
    d_base, d_lora, dg, _ = bnd.dora_compose_backward(dev(dy, "bf16"), dev(base, "bf16"), dev(lora, "bf16"), ones, s)
    # g = 1: no base gradient; d_lora = s * dy exactly (s is a power of two)
    assert torch.count_nonzero(d_base.float()) == 0
    assert torch.equal(d_lora.float().cpu(), torch.from_numpy(dy * np.float32(s)))
    gt = torch.from_numpy(g).cuda()
    a = bnd.dora_compose_backward(dev(dy, "bf16"), dev(base, "bf16"), dev(lora, "bf16"), gt, s)[2]
    b = bnd.dora_compose_backward(dev(dy, "bf16"), dev(base, "bf16"), dev(lora, "bf16"), gt, s)[2]
    assert torch.equal(a, b)


def test_compose_backward_unaligned_and_empty():
    T, d_out, s = 16, 512, 0.25
    dy, base, lora, g = _inputs(T, d_out, "bf16", 13)
    flat = torch.zeros(T * d_out + 1, dtype=torch.bfloat16, device="cuda")
    dy_un = flat[1:].view(T, d_out)
    dy_un.copy_(dev(dy, "bf16"))
    d_base, d_lora, dg, _ = bnd.dora_compose_backward(dy_un, dev(base, "bf16"), dev(lora, "bf16"),
                                                      torch.from_numpy(g).cuda(), s)
    rb, rl, rg = O.compose_backward(dy, base, lora, g, s)
    _check_elem(d_base, rb, "bf16", "d_base")
    _check_elem(d_lora, rl, "bf16", "d_lora")
    _check_dg(dg, dy, base, lora, s, rg)
    # T = 0: dg is an empty sum
    z = torch.zeros(0, d_out, dtype=torch.bfloat16, device="cuda")
    _, _, dg0, _ = bnd.dora_compose_backward(z, z, z, torch.from_numpy(g).cuda(), s)
    assert torch.count_nonzero(dg0) == 0


def test_compose_backward_argument_errors():
    T, d_out = 8, 64
    dy = torch.zeros(T, d_out, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(d_out, dtype=torch.float32, device="cuda")
    with pytest.raises(bnd.DoraError):
        bnd.dora_compose_backward(dy, dy, dy, g, 0.5, d_base=dy)   # output aliases an input
    with pytest.raises(bnd.DoraError):
        bnd.dora_compose_backward(dy, dy, dy, g, float("nan"))


def _backward_sweep():
    """Seeded shapes across the backward's strip grid: widths giving 1 to
    several column blocks, narrow workgroups with 2 and 4 row lanes, widths
    off the 16-byte vector (the element path), row counts from one row to
    thousands, trained and frozen magnitude."""
    rng = np.random.default_rng(919)
    out = []
    for k in range(20):
        dtype = ["bf16", "f16", "f32", "bf16"][k % 4]
        q = 4 if dtype == "f32" else 8
        d_out = int(rng.choice([rng.integers(1, 520), rng.integers(520, 5000)]))
        if k % 4 != 3:
            d_out = max(q, d_out // q * q)
        T = int(rng.choice([rng.integers(1, 9), rng.integers(9, 600), rng.integers(600, 2500)]))
        s = float(rng.choice([0.5, -0.75, 2.0]))
        out.append((T, d_out, dtype, s, k % 5 == 4))
    return out


BWD_SWEEP = _backward_sweep()


@pytest.mark.parametrize("k", range(len(BWD_SWEEP)))
def test_compose_backward_seeded_sweep(k):
    T, d_out, dtype, s, frozen = BWD_SWEEP[k]
    say(f"[compose-bwd-sweep] {k}: T={T} d_out={d_out} {dtype} s={s} frozen={frozen}")
    dy, base, lora, g = _inputs(T, d_out, dtype, 600 + k)
    _, wnorm = I.grad_inputs(T, d_out, dtype, 600 + k)
    if frozen:
        d_base, d_lora, dg, dm = bnd.dora_compose_backward(dev(dy, dtype), dev(base, dtype), dev(lora, dtype),
                                                           torch.from_numpy(g).cuda(), s, need_dg=False)
    else:
        d_base, d_lora, dg, dm = bnd.dora_compose_backward(dev(dy, dtype), dev(base, dtype), dev(lora, dtype),
                                                           torch.from_numpy(g).cuda(), s,
                                                           wnorm=torch.from_numpy(wnorm).cuda(), eps=1e-6)
    torch.cuda.synchronize()
    rb, rl, rg, rm = O.compose_backward(dy, base, lora, g, s, wnorm=wnorm, eps=1e-6)
    _check_elem(d_base, rb, dtype, "d_base")
    _check_elem(d_lora, rl, dtype, "d_lora")
    if frozen:
        assert dg is None and dm is None
    else:
        _check_dg(dg, dy, base, lora, s, rg)
        got_dm = dm.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(got_dm, O.magnitude_scale(dg.cpu().numpy().astype(np.float64), wnorm, 1e-6),
                                   rtol=2 * U32, atol=0)
