"""bench.py on the CPU: the one-GPU rule and the algorithmic work it reports."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_work_figures():
    # 8192 x 8192, r = 384, bf16, T = 8192
    assert round(bench.norm_flops(8192, 8192, 384) / 1e9, 1) == 56.5
    assert round(bench.norm_bytes(8192, 8192, 384, 2) / 1e6, 1) == 146.9
    assert round(bench.compose_bytes(8192, 8192, 2) / 1e6, 1) == 402.7
    plan = {"gram_term_fused": 1, "gram_folded": 0}
    assert round(bench.w_pass_flops(8192, 8192, 384, plan) / 1e9, 1) == 54.1
    # the W pass alone never exceeds the whole call's work
    for fused, folded in [(1, 0), (0, 1), (0, 0)]:
        p = {"gram_term_fused": fused, "gram_folded": folded}
        assert bench.w_pass_flops(4096, 4096, 64, p) <= bench.norm_flops(4096, 4096, 64)


@pytest.mark.parametrize("chunk", [64, 128, 1000])
def test_eager_factored_norm_baseline_is_the_row_norm(chunk):
    # The eager baseline of the whole-layer comparison (fp32 torch on the
    # CPU here) against the dense row norm of W + s B A formed in fp64:
    # chunks that split d_in unevenly, one chunk past d_in, and s < 0.
    import numpy as np
    import torch

    rng = np.random.default_rng(5)
    W = rng.standard_normal((37, 300))
    A = rng.standard_normal((11, 300)) * 0.2
    B = rng.standard_normal((37, 11)) * 0.2
    for s in (0.7, -1.3):
        ref = np.linalg.norm(W + s * (B @ A), axis=1)
        got = bench.eager_factored_norm(*(torch.tensor(v, dtype=torch.float32) for v in (W, A, B)), s, chunk)
        assert np.abs(got.numpy() - ref).max() <= 1e-5 * ref.max()
