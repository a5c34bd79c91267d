"""dora_factored_norm_noalloc: the norm for callers that cannot allocate.

Called through the C ABI and checked against dora_factored_norm (the
allocating entry point) on the same inputs: bitwise equal, since both run
the same plan and kernels, and within the norm's 1e-5 of the fp64 oracle.
Two calls in a row, the second smaller, so the second reads a scratch array
that still holds the first call's partial sums.
"""

import ctypes

import numpy as np
import pytest
import torch

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I
from oracle import dora_oracle as O

from gpu_helpers import check_g, check_norm, dev, say

EPS = 1e-6
P = ctypes.c_void_p


def test_noalloc_refuses_plans_beyond_its_scratch():
    """Host-only: a plan that cannot fit the 32 MiB scratch (the reduced Gram
    matrix alone of r = 4096 is 64 MiB) returns DORA_ERR_BUDGET before any
    HIP call, so this runs without a GPU."""
    lib = bnd.load()
    st = lib.dora_factored_norm_noalloc(P(0x100000), P(0x200000), P(0x300000), 0, 64, 4096, 4096, 0.5, 1 << 30,
                                        P(0x400000), None, 1e-6, None, None)
    assert st == 3
    assert lib.dora_factored_norm_noalloc(P(0x100000), P(0x200000), P(0x300000), 0, 64, 64, 8, float("nan"),
                                          1 << 28, P(0x400000), None, 1e-6, None, None) == 1
    assert lib.dora_factored_norm_noalloc(None, P(0x200000), P(0x300000), 0, 64, 64, 8, 0.5, 1 << 28,
                                          P(0x400000), None, 1e-6, None, None) == 1


@pytest.mark.gpu
def test_noalloc_matches_allocating_entry_point():
    lib = bnd.load()
    stream = torch.cuda.current_stream()
    # the headline rank (Gram pass, reduction, W pass with the Gram term,
    # assembly), then a smaller, ragged shape with G folded into the W pass
    for d_out, d_in, r, s, seed in [(1024, 4096, 384, 0.5, 61), (300, 1000, 72, 2.0, 62)]:
        say(f"    noalloc: {d_out}x{d_in} r={r}")
        W, A, B = I.norm_inputs(d_out, d_in, r, "bf16", seed)
        ref = O.dense_row_norm(W, A, B, s)
        m = (ref * (1.0 + I.G_SPREAD * I.m_noise(d_out, seed))).astype(np.float32)
        Wd, Ad, Bd = dev(W, "bf16"), dev(A, "bf16"), dev(B, "bf16")
        md = torch.from_numpy(m).cuda()
        wn_a, g_a = bnd.dora_factored_norm(Wd, Ad, Bd, s, m=md, eps=EPS)
        wn_b = torch.full((d_out,), float("nan"), device="cuda")
        g_b = torch.full((d_out,), float("nan"), device="cuda")
        st = lib.dora_factored_norm_noalloc(P(Wd.data_ptr()), P(Ad.data_ptr()), P(Bd.data_ptr()), 0, d_out, d_in, r,
                                            s, 256 << 20, P(wn_b.data_ptr()), P(md.data_ptr()), EPS,
                                            P(g_b.data_ptr()), P(stream.cuda_stream))
        assert st == 0, bnd.dora_status_string(st)
        torch.cuda.synchronize()
        a, b = wn_a.cpu().numpy(), wn_b.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(g_a.cpu().numpy().view(np.uint32), g_b.cpu().numpy().view(np.uint32))
        check_norm(b, ref)
        check_g(g_b.cpu().numpy(), m, ref, EPS)
