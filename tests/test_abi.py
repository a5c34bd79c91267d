"""C ABI checks that need no GPU: symbols, host planner, argument errors.

Every call here returns before anything is enqueued (host-only entry points,
or argument checks that fail), so no HIP device is touched.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from dora_weight_norm_amd import binding as bnd
from dora_weight_norm_amd import inputs as I
from oracle import dora_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MiB = 1 << 20

pytestmark = pytest.mark.skipif(not os.path.exists(bnd.LIB_PATH), reason="libdora.so not built")


def _declared():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"\b(dora_\w+)\s*\(", txt)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = bnd.load()
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert bnd.dora_version() == 10000
    for st in range(6):
        assert bnd.dora_status_string(st)


@pytest.mark.parametrize("d_out,d_in,budget", [
    (8192, 8192, 256 * MiB), (28672, 8192, 256 * MiB), (512, 3584, 256 * MiB), (4096, 4096, MiB),
    (100, 40, 256 * MiB), (1000, 8192, 700_000), (1, 1, 0), (0, 10, 5), (7, 0, 5), (3, 1 << 20, 1 << 40),
])
def test_chunk_size_matches_oracle_rule(d_out, d_in, budget):
    assert bnd.dora_norm_chunk_size(d_out, d_in, budget) == O.chunk_size(d_out, d_in, budget)


def dense_rule(d_out, d_in, r, dtype):
    """The documented choice of the dense fused pass: 16-bit storage, r >= d_out (or r > d_in with
    at most 4096 rows), d_in and r in whole 16-byte chunks, and A (and 64 rows of W or B) under
    2^31 bytes."""
    cheaper = r >= d_out or (r > d_in and d_out <= 4096)
    return (dtype in ("bf16", "f16") and cheaper and d_in % 8 == 0 and r % 8 == 0
            and r * d_in * 2 < 2 ** 31 and 64 * d_in * 2 < 2 ** 31 and 64 * r * 2 < 2 ** 31)


@pytest.mark.parametrize("name", sorted(I.WORKLOADS))
def test_plans_of_the_workloads(name):
    w = I.WORKLOADS[name]
    info = bnd.dora_norm_plan_info(w.d_out, w.d_in, w.r, w.dtype, w.s, w.budget)
    dense = dense_rule(w.d_out, w.d_in, w.r, w.dtype)
    assert info["mode"] == (3 if dense else 2)
    if dense:
        # one 64 x 128 tile per workgroup; the W pass fields describe the factored fallback
        assert info["dense_row_tiles"] == -(-w.d_out // 64) and info["dense_col_tiles"] == -(-w.d_in // 128)
        assert info["w_launch"] == 0
        return
    assert info["dense_row_tiles"] == 0 and info["dense_col_tiles"] == 0
    assert info["workspace_bytes"] <= w.budget
    assert info["workspace_bytes"] == bnd.dora_norm_workspace_size(w.d_out, w.d_in, w.r, w.dtype, w.s, w.budget)
    assert info["gram_grid"] <= 256 and info["lds_bytes"] <= 160 * 1024
    # the W pass: one workgroup per (row tile, d_in range)
    assert info["w_grid"] == -(-w.d_out // info["tile_rows"]) * info["col_tiles"] * info["w_ranges"]
    # square Gram tiles (128 x 128, or 64 x 64 where 8 ranges of their upper
    # triangle fit the chip) are the symmetric ones
    square = info["gram_fast_cfg"] in (1, 10)
    assert info["gram_symmetric"] == (square and w.dtype != "f32")
    if info["gram_symmetric"]:
        nt = info["gram_col_tiles"]
        assert nt * info["gram_tile_cols"] == -(-w.r // 128) * 128
        tiles_g = nt * (nt + 1) // 2
        n64 = 2 * -(-w.r // 128)
        assert (info["gram_tile_cols"] == 64) == (w.r > 64 and n64 * (n64 + 1) // 2 * 8 <= 256)
    else:
        tiles_g = -(-w.r // 128) * info["gram_col_tiles"]
    assert info["gram_grid"] == tiles_g * info["gram_ranges"]
    assert info["tile_cols"] * info["col_tiles"] >= w.r
    # the Gram term runs inside the W pass unless G is folded into it
    assert info["gram_term_fused"] == int(not info["gram_folded"])
    # launch order: [Gram pass, gram_reduce,] W pass, ...
    assert info["w_launch"] == (0 if info["gram_folded"] else 2)
    # the W pass with the Gram term runs in the die grid of two range groups
    # (by four row groups) where its ranges and row tiles divide evenly, of
    # four range groups (by two row groups) when its grid runs in several
    # rounds and they fit; the plan query has replayed its order on the host
    # (every tile once)
    n_mt = -(-w.d_out // info["tile_rows"])
    assert info["die_groups"] == die_groups_rule(info["w_ranges"], n_mt, info["col_tiles"], info["gram_folded"])


def die_groups_rule(xw, n_mt, n_nt, folded):
    if folded:
        return 0
    if xw * n_mt * n_nt > 256 and xw % 4 == 0 and n_mt % 2 == 0:
        return 4
    return 2 if xw % 2 == 0 and n_mt % 4 == 0 else 0


def test_plan_self_check_on_many_shapes():
    rng = np.random.default_rng(0)
    shapes = [(1, 1, 1), (1, 64, 1), (33, 65, 7), (256, 256, 8), (512, 3584, 768), (4096, 4096, 64),
              (8192, 8192, 384), (28672, 8192, 512), (8192, 8192, 768), (640, 1024, 1000), (5, 100000, 3)]
    shapes += [tuple(int(v) for v in (rng.integers(1, 5000), rng.integers(1, 9000), rng.integers(1, 1100)))
               for _ in range(40)]
    for (d_out, d_in, r) in shapes:
        for dt in ("bf16", "f32", "f16"):
            # (the query replays the W pass's workgroup order on the host and
            # fails unless it covers every tile exactly once)
            info = bnd.dora_norm_plan_info(d_out, d_in, r, dt, 0.5, 256 * MiB)
            assert info["die_groups"] in (0, 2, 4)
            if info["mode"] in (2, 3):
                n_mt = -(-d_out // info["tile_rows"])
                assert info["die_groups"] == die_groups_rule(info["w_ranges"], n_mt, info["col_tiles"],
                                                             info["gram_folded"]), (d_out, d_in, r, dt)
            assert info["mode"] == (3 if dense_rule(d_out, d_in, r, dt) else 2), (d_out, d_in, r, dt)
            assert info["tile_cols"] * info["col_tiles"] >= r
            if info["mode"] == 3:
                assert info["dense_row_tiles"] * 64 >= d_out and info["dense_col_tiles"] * 128 >= d_in


def test_w_pass_tile_shapes():
    # (d_out, d_in, r) -> (tile rows, tile columns, column tiles) of the bf16
    # W pass: one column tile up to r = 256, in 256-row tiles once there are
    # at least 32 of them and d_in >= 8192; 256-row tiles of 192 or 256
    # columns above, whichever pads r less
    expect = {(8192, 8192, 64): (256, 64, 1), (8192, 8192, 128): (256, 128, 1), (8192, 8192, 8): (256, 64, 1),
              (8192, 8191, 64): (128, 64, 1), (8192, 4096, 128): (128, 128, 1), (28672, 2048, 256): (128, 256, 1),
              (4096, 8192, 64): (128, 64, 1), (4096, 8192, 128): (128, 128, 1), (4096, 8192, 256): (128, 256, 1),
              (7936, 8192, 256): (128, 256, 1), (7937, 8192, 256): (256, 256, 1), (8192, 8192, 160): (256, 256, 1),
              (8192, 4096, 384): (256, 192, 2), (512, 3584, 384): (256, 192, 2), (8192, 4096, 512): (256, 256, 2),
              (8192, 4096, 768): (256, 192, 4), (8192, 4096, 1000): (256, 256, 4), (8192, 4096, 1100): (256, 192, 6)}
    for (d_out, d_in, r), shape in expect.items():
        info = bnd.dora_norm_plan_info(d_out, d_in, r, "bf16", 0.5, 256 * MiB)
        assert (info["tile_rows"], info["tile_cols"], info["col_tiles"]) == shape, (d_out, d_in, r)


def test_trivial_modes_need_no_workspace():
    assert bnd.dora_norm_plan_info(0, 10, 4, "bf16", 1.0)["mode"] == 0
    for args in [(10, 20, 4, "bf16", 0.0), (10, 20, 0, "bf16", 1.0), (10, 0, 4, "f32", 1.0)]:
        info = bnd.dora_norm_plan_info(*args)
        assert info["mode"] == 1 and info["workspace_bytes"] == 0


def test_budget_fallback_and_error():
    full = bnd.dora_norm_plan_info(8192, 8192, 384, "bf16", 0.5, 256 * MiB)
    small = bnd.dora_norm_plan_info(8192, 8192, 384, "bf16", 0.5, 2 * MiB)
    assert small["workspace_bytes"] <= 2 * MiB < full["workspace_bytes"]
    assert small["gram_ranges"] < full["gram_ranges"]
    with pytest.raises(bnd.DoraError) as e:
        bnd.dora_norm_workspace_size(8192, 8192, 384, "bf16", 0.5, 1024)
    assert e.value.status == 3


def _raw_norm(**kw):
    a = dict(W=0x100000, A=0x200000, B=0x300000, dtype=0, d_out=16, d_in=32, r=4, s=0.5,
             budget=256 * MiB, ws=None, ws_bytes=0, wnorm=0x400000, m=None, eps=1e-6, g=None)
    a.update(kw)
    lib = bnd.load()
    P = ctypes.c_void_p
    return lib.dora_factored_norm(P(a["W"]), P(a["A"]), P(a["B"]), a["dtype"], a["d_out"], a["d_in"], a["r"],
                                  a["s"], a["budget"], P(a["ws"]), a["ws_bytes"], P(a["wnorm"]), P(a["m"]),
                                  a["eps"], P(a["g"]), None)


def test_norm_argument_errors_return_before_launch():
    assert _raw_norm(dtype=7) == 2
    assert _raw_norm(d_out=-1) == 1
    assert _raw_norm(s=float("nan")) == 1
    assert _raw_norm(m=0x500000, g=0x600000, eps=0.0) == 1
    assert _raw_norm(m=0x500000, g=None) == 1
    assert _raw_norm(wnorm=None) == 1
    assert _raw_norm(A=None) == 1
    assert _raw_norm(wnorm=0x100010) == 1                  # output inside W
    assert _raw_norm(W=0x100001) == 1                      # misaligned element
    assert _raw_norm(d_out=8192, d_in=8192, r=384, budget=1024) == 3
    assert _raw_norm(ws=None, ws_bytes=0) == 4             # workspace required
    assert _raw_norm(d_out=0) == 0                         # nothing to do


def test_compose_argument_errors_return_before_launch():
    lib = bnd.load()
    P = ctypes.c_void_p

    def call(base=0x100000, lora=0x200000, g=0x300000, s=0.5, dtype=0, T=4, d_out=8, out=0x400000):
        return lib.dora_compose(P(base), P(lora), P(g), s, dtype, T, d_out, P(out), None)

    assert call(dtype=9) == 2
    assert call(T=-1) == 1
    assert call(s=float("inf")) == 1
    assert call(base=None) == 1
    assert call(out=0x100002) == 1          # partial overlap with base
    assert call(out=0x300000 - 4) == 1      # overlaps g
    assert call(T=0) == 0 and call(d_out=0) == 0


def test_magnitude_argument_errors():
    lib = bnd.load()
    P = ctypes.c_void_p
    assert lib.dora_magnitude_scale(P(0x1000), P(0x2000), 0.0, 4, P(0x3000), None) == 1
    assert lib.dora_magnitude_scale(P(0x1000), P(0x2000), 1e-6, -1, P(0x3000), None) == 1
    assert lib.dora_magnitude_scale(None, None, 1e-6, 0, None, None) == 0
    assert lib.dora_magnitude_scale(P(0x1000), P(0x1004), 1e-6, 4, P(0x1004), None) == 1   # g overlaps m


def test_library_resolves_every_kernel_stub():
    """The host pass of hipcc can drop a kernel's launch stub without an error;
    the library then fails to load. Every kernel stub must be defined."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", bnd.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "device_stub" not in out, [ln for ln in out.splitlines() if "device_stub" in ln][:5]


def test_layer_output_argument_errors_return_before_launch():
    lib = bnd.load()
    P = ctypes.c_void_p

    def call(base=0x100000, lora=0x200000, g=0x300000, s=0.5, dtype=0, T=4, d_out=8, y=0x400000):
        return lib.dora_layer_output(P(base), P(lora), P(g), s, dtype, T, d_out, P(y), None)

    assert call(dtype=3) == 2                # 0 bf16, 1 fp32, 2 fp16; nothing else
    assert call(T=-1) == 1
    assert call(s=float("nan")) == 1
    assert call(lora=None) == 1
    assert call(y=0x200002) == 1             # partial overlap with lora
    assert call(y=0x100001) == 1             # misaligned element
    assert call(T=0) == 0 and call(d_out=0) == 0


def test_norm_to_dtype_argument_errors():
    lib = bnd.load()
    P = ctypes.c_void_p
    assert lib.dora_norm_to_dtype(P(0x1000), 8, 5, P(0x2000), None) == 2
    assert lib.dora_norm_to_dtype(P(0x1000), -1, 0, P(0x2000), None) == 1
    assert lib.dora_norm_to_dtype(None, 8, 0, P(0x2000), None) == 1
    assert lib.dora_norm_to_dtype(P(0x1002), 8, 0, P(0x2000), None) == 1     # wnorm misaligned
    assert lib.dora_norm_to_dtype(P(0x1000), 8, 0, P(0x2001), None) == 1     # bf16 out misaligned
    assert lib.dora_norm_to_dtype(P(0x1000), 8, 0, P(0x1010), None) == 1     # out overlaps wnorm
    assert lib.dora_norm_to_dtype(None, 0, 0, None, None) == 0               # nothing to do


def test_marked_norm_event_arguments():
    """The timing variant refuses a negative event count or a missing event
    array before doing anything else (argument errors return before launch)."""
    lib = bnd.load()
    P = ctypes.c_void_p
    args = (P(0x100000), P(0x200000), P(0x300000), 0, 64, 64, 8, 0.5, 1 << 28, P(0x400000), 1 << 20,
            P(0x500000), None, 1e-6, None, None)
    assert lib.dora_factored_norm_marked(*args, None, -1) == 1
    assert lib.dora_factored_norm_marked(*args, None, 2) == 1
    bad = list(args)
    bad[4] = -1                                                 # negative d_out, no events
    assert lib.dora_factored_norm_marked(*bad, None, 0) == 1


def test_streaming_offsets_guard_uses_the_tallest_tile():
    """The streaming kernel's 32-bit descriptor offsets: every operand tile
    (the W pass's 256-row tiles included) must span less than 2^31 bytes,
    else the general kernel runs. 256 rows x 5M bf16 elements is 2.56 GB."""
    ok = bnd.dora_norm_plan_info(8192, 8192, 64, "bf16", 0.5)
    assert ok["tile_rows"] == 256 and ok["offsets32"] == 1
    big = bnd.dora_norm_plan_info(8192, 5 << 20, 64, "bf16", 0.5, budget_bytes=1 << 34)
    assert big["tile_rows"] == 256 and big["offsets32"] == 0
    # 128-row tiles: just under 4M elements fit (about 2^30 bytes); 8M (2^31 bytes) do not
    edge = bnd.dora_norm_plan_info(4096, (1 << 22) - 64, 64, "bf16", 0.5, budget_bytes=1 << 34)
    assert edge["tile_rows"] == 128 and edge["offsets32"] == 1
    over = bnd.dora_norm_plan_info(4096, 1 << 23, 64, "bf16", 0.5, budget_bytes=1 << 34)
    assert over["offsets32"] == 0


def test_compose_backward_argument_errors_return_before_launch():
    lib = bnd.load()
    P = ctypes.c_void_p
    sz = ctypes.c_size_t()
    assert lib.dora_compose_backward_workspace_size(4, 8, ctypes.byref(sz)) == 0 and sz.value > 0
    assert lib.dora_compose_backward_workspace_size(-1, 8, ctypes.byref(sz)) == 1
    assert lib.dora_compose_backward_workspace_size(4, 8, None) == 1

    def call(dy=0x100000, base=0x200000, lora=0x300000, g=0x400000, s=0.5, dtype=0, T=4, d_out=8,
             d_base=0x500000, d_lora=0x600000, dg=0x700000, wnorm=None, eps=1e-6, dm=None, ws=0x800000,
             ws_bytes=1 << 20):
        return lib.dora_compose_backward(P(dy), P(base), P(lora), P(g), s, dtype, T, d_out, P(d_base), P(d_lora),
                                         P(dg), P(wnorm), eps, P(dm), P(ws), ws_bytes, None)

    assert call(dtype=4) == 2
    assert call(T=-1) == 1
    assert call(s=float("inf")) == 1
    assert call(dy=None) == 1
    assert call(base=None) == 1                        # dg needs base and lora
    assert call(dm=0x900000) == 1                      # dm needs wnorm
    assert call(dm=0x900000, wnorm=0xA00000, eps=0.0) == 1
    assert call(d_lora=0x500010) == 1                  # outputs overlap
    assert call(d_base=0x100000) == 1                  # output is an input
    assert call(ws_bytes=16) == 4                      # workspace too small
    assert call(d_out=0) == 0


def test_no_kernel_uses_scratch_or_spills_vector_registers():
    # build() records the compiler's per-kernel resource use; a scratch array
    # or spilled vector registers would put every access on memory.
    from dora_weight_norm_amd import build as B
    if not os.path.exists(B.RESOURCE_REPORT):
        pytest.skip("no build report (run build() first)")
    rows = {}
    for ln in open(B.RESOURCE_REPORT):
        name, *fields = ln.split()
        rows[name] = dict(f.split("=", 1) for f in fields)
    assert rows
    for name, d in rows.items():
        assert d["ScratchSize_[bytes/lane]"] == "0", name
        assert d["VGPRs_Spill"] == "0", name
    def find(pat):
        return [d for n, d in rows.items() if pat in n]
    # the 256 x 384 W-pass tile (bf16, Gram term inside): 192 accumulators
    # per lane at two waves per SIMD, so at most 256 registers in all
    lean = find("norm_fast_kernelItLi2ELi4ELi4ELi3ELi64ELi2ELi4E")
    assert lean and all(int(d["VGPRs"]) + int(d["AGPRs"]) <= 256 and d["Occupancy_[waves/SIMD]"] == "2"
                        for d in lean)
    assert find("norm_dense_kernel") and find("compose_kernel") and find("compose_bwd_kernel")


def test_die_grid_edge_shapes_plan_as_the_gpu_cases_assume():
    # tests/test_gpu_norm.py runs these shapes for the die grid's edges:
    # two d_in ranges (one per range group) with several column tiles, and
    # four ranges with one column tile
    two = bnd.dora_norm_plan_info(7168, 512, 768, "bf16", 0.5, 256 * MiB)
    assert two["mode"] == 2 and two["die_groups"] == 2 and two["w_ranges"] == 2 and two["col_tiles"] > 1
    four = bnd.dora_norm_plan_info(8192, 512, 192, "bf16", -0.25, 256 * MiB)
    assert four["mode"] == 2 and four["die_groups"] == 2 and four["w_ranges"] == 4 and four["col_tiles"] == 1
    # grids of several rounds, the last one partial, in four range groups
    # (by two row groups), with 192- and 256-column tiles; the 28672 x 8192,
    # r = 512 workload plans the same way
    multi = bnd.dora_norm_plan_info(4608, 1024, 384, "bf16", 0.5, 256 * MiB)
    assert multi["mode"] == 2 and multi["die_groups"] == 4 and multi["col_tiles"] == 2
    assert multi["w_grid"] % 256 != 0 and multi["w_grid"] > 512 and multi["w_ranges"] == 16
    assert multi["tile_cols"] == 192
    wide = bnd.dora_norm_plan_info(8704, 512, 448, "bf16", -0.5, 256 * MiB)
    assert wide["mode"] == 2 and wide["die_groups"] == 4 and wide["col_tiles"] == 2
    assert wide["tile_cols"] == 256 and wide["w_grid"] > 256 and wide["w_ranges"] == 8
    mlp = bnd.dora_norm_plan_info(28672, 8192, 512, "bf16", 0.5, 256 * MiB)
    assert mlp["die_groups"] == 4 and mlp["w_grid"] > 256
