"""The library's kernel table: every kernel's LDS budget adds up and fits one
gfx950 compute unit (CPU); the compiled kernels declare exactly the LDS the
table states (GPU).

The shared-memory budget of a pipelined GEMM is stages x bytes per stage plus
the fixed buffers beside the ring; a budget that leaves a buffer out silently
changes the occupancy and the stage count the kernel can afford ([W4A4] page,
"最新GPU架构上W4A4算子的Warp专用化内核实践", §6)."""

import os

import pytest

import fp4_grouped_gemm_amd as fgg

LDS_PER_CU = 160 * 1024

pytestmark = pytest.mark.skipif(not os.path.exists(fgg.library_path()),
                                reason="libfgg.so not built (run __graft_entry__.build())")


def test_table_lists_every_kernel_once():
    t = fgg.kernel_table()
    names = [k["kernel"] for k in t]
    assert len(names) == len(set(names))
    for required in ("gemm_fp8_contig_kernel<plain>", "gemm_fp8_contig_kernel<silu>", "gemm_fp8_dense_kernel",
                     "gemm_masked_fp4_lds_kernel<tiled>", "w4a4_gemm_kernel", "permute_scatter_kernel",
                     "permute_quantize_kernel", "combine_kernel"):
        assert required in names, required
    for k in t:
        assert k["entry"].startswith("fgg_"), k


def test_budget_arithmetic_and_limits():
    for k in fgg.kernel_table():
        assert k["stages"] * k["stage_bytes"] + k["other_bytes"] == k["lds_bytes"], k
        assert 0 <= k["lds_bytes"] <= LDS_PER_CU, k
        assert k["threads"] % 64 == 0 and 64 <= k["threads"] <= 1024, k
        assert k["stages"] == 0 or k["stage_bytes"] > 0, k


def test_gemm_rings_hold_their_tiles():
    """Each GEMM stage holds the A and B tile bytes of one K step (plus its scales)."""
    t = {k["kernel"]: k for k in fgg.kernel_table()}
    for name in ("gemm_fp8_contig_kernel<plain>", "gemm_fp8_contig_kernel<silu>", "gemm_fp8_dense_kernel"):
        k = t[name]
        tile_bytes = (k["tile_m"] + k["tile_n"]) * k["tile_k"]          # e4m3: one byte per element
        assert k["stage_bytes"] >= tile_bytes + 4 * k["tile_m"], k      # + the activation scales
    k = t["w4a4_gemm_kernel"]
    assert k["stage_bytes"] == (k["tile_m"] + k["tile_n"]) * k["tile_k"] * 2      # fp16 operands


def test_bad_index_is_rejected():
    import ctypes
    lib = fgg.load_library()
    info = fgg.KernelInfo()
    n = lib.fgg_kernel_count()
    assert lib.fgg_kernel_info_get(n, ctypes.byref(info)) == 1
    assert lib.fgg_kernel_info_get(-1, ctypes.byref(info)) == 1
    assert lib.fgg_kernel_info_get(0, None) == 1


@pytest.mark.gpu
def test_compiled_lds_matches_table():
    for i, k in enumerate(fgg.kernel_table()):
        assert fgg.kernel_compiled_lds(i) == k["lds_bytes"], k
