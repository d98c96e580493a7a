"""Host-side pieces of the benchmark (no GPU): the profile summarizers' parsing."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_short_kernel_name():
    f = bench._short_kernel_name
    assert f("hypic::(anonymous namespace)::gdn_build_mfma_kernel(hypic::BuildArgs)") == "gdn_build_mfma_kernel"
    assert (f("void hypic::(anonymous namespace)::compose_dense_mfma_kernel<false, true>(hypic::ComposeArgs)")
            == "compose_dense_mfma_kernel<false, true>")
    assert f("void (anonymous namespace)::peak_read_kernel(float const*, long, float*)") == "peak_read_kernel"
    # a parenthesis inside the template arguments is not the parameter list
    assert f("void k<(unsigned char)1, 2>(int)") == "k<(unsigned char)1, 2>"


def test_every_traced_workload_has_a_trace_key():
    for (name, grid), title in bench.TRACE_WORKLOADS.items():
        assert bench._trace_key(name) == name and grid > 0 and title

