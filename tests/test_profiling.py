"""Host logic of the profile summaries bench.py reads its measured traffic
from: the code hash that ties counters to kernel code, kernel naming, the
copy calibration, and the committed summaries' shape."""

import glob
import json
import os

import pytest

from dora_weight_norm_amd import inputs as I
from dora_weight_norm_amd import profiling as prof

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_hash_ignores_comments_but_not_code():
    a = 'int x = 1;  // one\nint y = 2;\n'
    b = 'int x = 1;  // one, reworded\n/* a new\n   block comment */\n\nint y = 2;   \n'
    c = 'int x = 3;  // one\nint y = 2;\n'
    assert prof._code_only(a) == prof._code_only(b) == "int x = 1;\nint y = 2;"
    assert prof._code_only(a) != prof._code_only(c)
    # comment markers inside literals are code
    s = 'const char* p = "a // b /* c */";\nchar q = \'/\';\n'
    assert prof._code_only(s) == s.rstrip("\n")


def test_source_hash_is_stable():
    h = prof.source_hash()
    assert len(h) == 16 and h == prof.source_hash()


def test_kernel_roles_and_short_names():
    ns = "void dora::(anonymous namespace)::"
    w = ns + "norm_fast_kernel<unsigned short, 4, 2, 2, 3, 64, 2, 4>(dora::NormPlan, unsigned short const*)"
    assert prof.kernel_role(w) == "norm"
    assert prof.short_name(w) == "norm_fast_kernel<bf16, 4, 2, 2, 3, 64, 2, 4> (W pass + Gram term)"
    g = ns + "norm_fast_kernel<unsigned short, 2, 4, 2, 1, 64, 4, 1>(dora::NormPlan, unsigned short const*)"
    assert prof.short_name(g).endswith("(Gram pass)")
    assert prof.kernel_role(ns + "compose_kernel<unsigned short, 8, false>(unsigned short const*)") == "compose"
    assert prof.kernel_role(ns + "compose_kernel<unsigned short, 8, true>(unsigned short const*)") == "layer_output"
    assert prof.kernel_role(ns + "compose_bwd_kernel<unsigned short, 8, true>(unsigned short const*)") == "compose_bwd"
    assert prof.kernel_role("__amd_rocclr_copyBuffer") is None
    d = ns + "norm_dense_kernel<unsigned short, 8>(dora::NormPlan, unsigned short const*)"
    assert prof.kernel_role(d) == "norm" and prof.short_name(d) == "norm_dense_kernel<bf16, 8> (dense pass)"
    assert prof.is_main_pass(d) and prof.is_main_pass(w) and not prof.is_main_pass(g)


def test_names_left_mangled_by_the_profiler():
    # rocprofv3 prints a name mangled when it holds _Float16 (DF16_); the
    # library's own names are decoded, others pass through
    red = "_ZN4dora12_GLOBAL__N_118gram_reduce_kernelItEEvNS_8NormPlanEPcfPKDF16_i"
    assert prof.demangle_ours(red) == "void dora::(anonymous namespace)::gram_reduce_kernel<unsigned short>()"
    assert prof.kernel_role(red) == "norm" and prof.short_name(red) == "gram_reduce_kernel<bf16>"
    w16 = ("_ZN4dora12_GLOBAL__N_116norm_fast_kernelIDF16_Li2ELi4ELi4ELi3ELi64ELi2ELi4EEEvNS_8NormPlanEPKT_S5_S5_"
           "PcNS0_12AssembleArgsE")
    assert prof.short_name(w16) == "norm_fast_kernel<f16, 2, 4, 4, 3, 64, 2, 4> (W pass + Gram term)"
    assert prof.is_main_pass(w16)
    lay = "_ZN4dora12_GLOBAL__N_114compose_kernelIDF16_Li8ELb1EEEvPKT_S4_PKffllPS2_"
    assert prof.kernel_role(lay) == "layer_output"
    assert prof.kernel_role("_ZN4dora12_GLOBAL__N_114compose_kernelIDF16_Li8ELb0EEEvPKT_") == "compose"
    other = "_ZN2at6native29vectorized_elementwise_kernelILi4EEEvi"
    assert prof.demangle_ours(other) == other and prof.kernel_role(other) is None


def test_copy_calibration():
    # a 1 GiB copy whose counter reads 512 MiB (in KiB) scales by 2
    per = {"__amd_rocclr_copyBuffer": [1024.0, 524288.0],
           "void dora::(anonymous namespace)::compose_kernel<unsigned short, 8, false>()": [9e9]}
    assert prof.calibration(per) == 2.0
    with pytest.raises(RuntimeError):
        prof.calibration({"void dora::x()": [1.0]})


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))),
                         ids=lambda p: os.path.basename(p))
def test_committed_traffic_summaries(path):
    d = json.load(open(path))
    assert d["workload"] in I.WORKLOADS
    assert os.path.basename(path) == f"traffic_{d['workload']}.json"
    assert len(d["source_hash"]) == 16
    for k in ("norm_bytes_per_call", "compose_bytes_per_call", "w_pass_bytes_per_launch",
              "norm_us_per_call", "compose_us_per_call"):
        assert d[k] > 0, k
    assert d["longest_step_kernel"]["part"] in ("norm", "compose")
    assert d["fetch_scale"] > 0 and d["write_scale"] > 0
    for cmd in d["commands"].values():
        assert cmd.startswith("rocprofv3 ") and " -- python bench.py " in cmd
    md = os.path.join(ROOT, "profiles", f"norm_compose_{d['workload']}.md")
    assert os.path.exists(md)
