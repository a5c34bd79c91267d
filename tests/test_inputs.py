"""The seeded generators: reproducible, storage-exact, independent streams."""

import numpy as np

from dora_weight_norm_amd import inputs as I


def test_reproducible_and_streams_independent():
    W1, A1, B1 = I.norm_inputs(64, 96, 8, "bf16", seed=5)
    W2, A2, B2 = I.norm_inputs(64, 96, 8, "bf16", seed=5)
    assert np.array_equal(W1, W2) and np.array_equal(A1, A2) and np.array_equal(B1, B2)
    # a different rank changes A and B only, never W
    W3, _, _ = I.norm_inputs(64, 96, 16, "bf16", seed=5)
    assert np.array_equal(W1, W3)
    W4, _, _ = I.norm_inputs(64, 96, 8, "bf16", seed=6)
    assert not np.array_equal(W1, W4)


def test_bf16_values_are_exact_and_rne():
    W, A, B = I.norm_inputs(32, 128, 8, "bf16", seed=1)
    for x in (W, A, B):
        assert x.dtype == np.float32
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)
    x64 = I.normal(1, "W", (32, 128), 1.0 / np.sqrt(128))
    x32 = x64.astype(np.float32)
    # RNE: the rounding error is at most half a bf16 ulp of the fp32 value
    ulp = np.ldexp(1.0, np.frexp(np.abs(x32.astype(np.float64)))[1] - 8)
    assert np.all(np.abs(W.astype(np.float64) - x32) <= ulp / 2)


def test_distributions():
    W, A, B = I.norm_inputs(512, 1024, 64, "bf16", seed=2)
    assert abs(W.std() * np.sqrt(1024) - 1.0) < 0.02
    assert abs(A.std() * np.sqrt(1024) - 1.0) < 0.03
    assert abs(B.std() / 0.02 - 1.0) < 0.03
    base, lora, g = I.compose_inputs(256, 1024, "bf16", seed=2)
    assert abs(base.std() - 1.0) < 0.02 and abs(lora.std() / 0.1 - 1.0) < 0.02
    assert g.dtype == np.float32 and abs(g.mean() - 1.0) < 3e-4 and abs(g.std() / 0.0015 - 1) < 0.1


def test_f32_storage_and_workloads():
    W, _, _ = I.norm_inputs(16, 16, 2, "f32", seed=0)
    assert W.dtype == np.float32 and np.any((W.view(np.uint32) & 0xFFFF) != 0)
    names = set(I.WORKLOADS)
    assert I.HEADLINE.name in names and len(names) == 6
    h = I.HEADLINE
    assert (h.d_out, h.d_in, h.r, h.s, h.dtype, h.T) == (8192, 8192, 384, 0.5, "bf16", 8192)
