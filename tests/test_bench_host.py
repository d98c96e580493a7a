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
    for (name, grid, phase), title in bench.TRACE_WORKLOADS.items():
        assert bench._trace_key(name) == name and (grid is None or grid > 0) and title
        assert phase in bench.PHASES


def test_tables_name_known_phases():
    for frag, grid, phase, sources, title in bench.TRAFFIC_KERNELS.values():
        assert phase in bench.PHASES and sources and title
    for frag, grid, phase, title, ty in bench.MFMA_KERNELS:
        assert phase in bench.PHASES and ty in ("BF16", "F32")


def test_dispatch_phases():
    """Every dispatch belongs to the phase of the last marker launch before it (in
    dispatch order, whatever the row order); markers are left out; dispatches before
    the first marker have none; the peak copy's own full-size launch is no marker."""
    code = {p: 512 * (i + 1) for i, p in enumerate(bench.PHASES)}
    rows = [(1, "__amd_rocclr_copyBuffer", 131072),
            (2, "void (anonymous namespace)::peak_copy_kernel(f32x4 const*, f32x4*, long)", code["main"]),
            (3, "hypic::gdn_build_mfma_kernel(hypic::BuildArgs)", 131072),
            (5, "hypic::gdn_build_mfma_kernel(hypic::BuildArgs)", 131072),
            (4, "peak_copy_kernel", code["rag"]),
            (6, "peak_copy_kernel", 8388608),
            (7, "peak_copy_kernel", code["peaks"]),
            (8, "peak_copy_kernel", 8388608)]
    ph = bench.dispatch_phases(rows)
    assert ph == {1: None, 3: "main", 5: "rag", 6: "rag", 8: "peaks"}
    # the trace workload lookup: exact grid first, then any grid
    assert bench._trace_workload("gdn_build_mfma_kernel", 131072, "rag") == ("gdn_build_mfma_kernel", None, "rag")
    assert bench._trace_workload("sd_build_mfma_kernel<0, 2>", 131072, "sd") == ("sd_build_mfma_kernel<0, 2>",
                                                                                 131072, "sd")
    assert bench._trace_workload("sd_build_mfma_kernel<0, 2>", 65536, "sd") is None
    assert bench._trace_workload("gdn_build_mfma_kernel", 131072, None) is None

