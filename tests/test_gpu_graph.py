"""A norm call and a compose captured into one HIP graph (torch.cuda.CUDAGraph)
and replayed.

With the workspace and the outputs passed in, neither call allocates device
memory, synchronises with the host or records a memset (the W pass's arrival
counters are cleared by a kernel of the same call), so a step can be captured
once and replayed. Each replay is compared bitwise with the eager calls on the
same inputs; between replays the program runs eager calls of its own, on
other inputs but the same workspace, so a replay must not depend on what an
earlier call left in it.
"""

import numpy as np
import pytest
import torch

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I

from gpu_helpers import dev, say

pytestmark = pytest.mark.gpu

EPS = 1e-6

# the factored path with the assembly in the W pass (one round), the dense
# pass (r >= d_out), the W pass with G folded in, a W pass of several rounds
# in four range groups (separate assembly launch), and fp16 with B split
CASES = [
    ("factored_assembly_in_w", 2048, 8192, 384, "bf16", 0.5),
    ("dense", 512, 3584, 768, "bf16", 0.25),
    ("gram_folded", 4096, 4096, 64, "bf16", -0.5),
    ("several_rounds", 4608, 1024, 384, "bf16", 0.5),
    ("f16_split_b", 1000, 1024, 384, "f16", 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(case):
    name, d_out, d_in, r, dtype, s = case
    say(f"[graph] {name} d_out={d_out} d_in={d_in} r={r} {dtype} s={s}")
    T = 256
    W, A, B = (dev(x, dtype) for x in I.norm_inputs(d_out, d_in, r, dtype, 11))
    W2, A2, B2 = (dev(x, dtype) for x in I.norm_inputs(d_out, d_in, r, dtype, 12))
    base_h, lora_h, _ = I.compose_inputs(T, d_out, dtype, 13)
    base, lora = dev(base_h, dtype), dev(lora_h, dtype)
    m = torch.from_numpy((1.0 + 0.01 * I.m_noise(d_out, 14)).astype(np.float32)).cuda()
    ws = torch.empty(max(bnd.dora_norm_workspace_size(d_out, d_in, r, dtype, s), 1), dtype=torch.uint8,
                     device="cuda")
    wn = torch.empty(d_out, device="cuda")
    g = torch.empty(d_out, device="cuda")
    out = torch.empty_like(base)
    st = torch.cuda.Stream()

    def step(Wx, Ax, Bx):
        bnd.dora_factored_norm(Wx, Ax, Bx, s, m=m, eps=EPS, workspace=ws, wnorm=wn, g=g, stream=st)
        bnd.dora_compose(base, lora, g, s, out=out, stream=st)

    with torch.cuda.stream(st):
        step(W, A, B)
    torch.cuda.synchronize()
    ref = (wn.clone(), g.clone(), out.clone())
    with torch.cuda.stream(st):
        step(W2, A2, B2)
    torch.cuda.synchronize()
    other = (wn.clone(), g.clone(), out.clone())
    assert not torch.equal(other[0], ref[0])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        step(W, A, B)
    torch.cuda.synchronize()
    for k in range(4):
        wn.fill_(float("nan"))
        g.fill_(float("nan"))
        out.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            graph.replay()
        torch.cuda.synchronize()
        for got, want, nm in zip((wn, g, out), ref, ("wnorm", "g", "out")):
            assert torch.equal(got, want), f"replay {k}: {nm} differs from the eager call"
        # eager work of the program between replays: other inputs, same workspace
        with torch.cuda.stream(st):
            step(W2, A2, B2)
        torch.cuda.synchronize()
        assert torch.equal(wn, other[0]) and torch.equal(out, other[2])
