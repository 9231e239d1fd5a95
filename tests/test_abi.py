"""CPU checks of the C ABI: libfgg.so loads, exports every function that
include/fgg.h declares, and rejects bad arguments on the host before any
device work (these calls return before touching HIP)."""

import ctypes
import os
import re

import pytest

import fp4_grouped_gemm_amd as fgg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fgg.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fgg.library_path()),
                                reason="libfgg.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["fgg_quantize_blockwise", "fgg_moe_permute", "fgg_moe_permute_workspace", "fgg_moe_permute_quantize",
              "fgg_grouped_gemm_scaled", "fgg_grouped_gemm_silu_quantize",
              "fgg_pack_fp4_weights_bytes", "fgg_pack_fp4_weights",
              "fgg_scaled_gemm", "fgg_scaled_gemm_workspace", "fgg_moe_combine", "fgg_moe_down_combine",
              "fgg_moe_down_combine_workspace", "fgg_status_string",
              "fgg_last_hip_error", "fgg_set_num_cus"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fgg.library_path())
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_knobs():
    lib = fgg.load_library()
    assert lib.fgg_status_string(0) == b"FGG_OK"
    assert lib.fgg_status_string(2) == b"FGG_ERR_UNSUPPORTED"
    assert lib.fgg_set_num_cus(-1) == 1
    assert lib.fgg_set_num_cus(0) == 0


def _q(t):
    return fgg.QDesc(*t)


def test_quantize_rejects_bad_arguments_on_host():
    lib = fgg.load_library()
    P = ctypes.c_void_p
    good = P(4096)
    # negative rows
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, -1, 128, 128, 0, _q(fgg.Q_E4M3_1x128), None, good, good, None) == 1
    # unsupported descriptor
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, 4, 128, 128, 0, _q((fgg.FGG_E4M3, fgg.FGG_F32, 1, 64)),
                                      None, good, good, None) == 2
    # cols not a multiple of the block
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, 4, 100, 128, 0, _q(fgg.Q_E4M3_1x128), None, good, good, None) == 2
    # 128-row blocks with a ragged row count
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, 100, 128, 128, 0, _q(fgg.Q_E4M3_128x128), None, good, good,
                                      None) == 2
    # SiLU only with the 1x128 e4m3 kind
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_BF16, 4, 32, 64, 1, _q(fgg.Q_E2M1_E8M0_1x32), None, good, good,
                                      None) == 2
    # null pointers / short leading dimension / misalignment
    assert lib.fgg_quantize_blockwise(None, fgg.FGG_F32, 4, 128, 128, 0, _q(fgg.Q_E4M3_1x128), None, good, good, None) == 1
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, 4, 256, 128, 0, _q(fgg.Q_E4M3_1x128), None, good, good, None) == 1
    assert lib.fgg_quantize_blockwise(P(4097), fgg.FGG_F32, 4, 128, 128, 0, _q(fgg.Q_E4M3_1x128), None, good,
                                      good, None) == 1
    # the device row limit only with the 1x128 e4m3 kind
    assert lib.fgg_quantize_blockwise(good, fgg.FGG_F32, 128, 128, 128, 0, _q(fgg.Q_E4M3_128x128), good, good,
                                      good, None) == 2
    # empty input is a successful no-op even without a device
    assert lib.fgg_quantize_blockwise(None, fgg.FGG_F32, 0, 128, 128, 0, _q(fgg.Q_E4M3_1x128), None, None, None, None) == 0


def test_gemm_and_permute_reject_bad_arguments_on_host():
    lib = fgg.load_library()
    P = ctypes.c_void_p
    g = P(4096)
    A, B8, B4 = _q(fgg.Q_E4M3_1x128), _q(fgg.Q_E4M3_128x128), _q(fgg.Q_E2M1_E8M0_1x32)
    # N not a multiple of 128
    assert lib.fgg_grouped_gemm_scaled(0, 2, 256, 100, 256, g, g, A, g, g, B8, g, None, g, 128, None) == 2
    # K not a multiple of 128
    assert lib.fgg_grouped_gemm_scaled(0, 2, 256, 128, 200, g, g, A, g, g, B8, g, None, g, 128, None) == 2
    # contiguous layout needs offsets; masked needs masked_m and M <= 16
    assert lib.fgg_grouped_gemm_scaled(0, 2, 256, 128, 256, g, g, A, g, g, B8, None, None, g, 128, None) == 1
    assert lib.fgg_grouped_gemm_scaled(1, 2, 16, 128, 256, g, g, A, g, g, B4, None, None, g, 128, None) == 1
    assert lib.fgg_grouped_gemm_scaled(1, 2, 17, 128, 256, g, g, A, g, g, B4, None, g, g, 128, None) == 2
    # FP4 weights are not a contiguous-layout operand
    assert lib.fgg_grouped_gemm_scaled(0, 2, 256, 128, 256, g, g, A, g, g, B4, g, None, g, 128, None) == 2
    # ldd smaller than N, bad G
    assert lib.fgg_grouped_gemm_scaled(0, 2, 256, 256, 256, g, g, A, g, g, B8, g, None, g, 128, None) == 1
    assert lib.fgg_grouped_gemm_scaled(0, 0, 256, 128, 256, g, g, A, g, g, B8, g, None, g, 128, None) == 1
    # dense W4A4 with an unsupported rank
    epi = fgg.Epilogue(4096, 4096, 4096, 16, None)
    W = _q(fgg.Q_E2M1_1x16)
    assert lib.fgg_scaled_gemm(256, 128, 256, g, g, W, g, g, W, ctypes.byref(epi), g, 128, g, 1 << 20, None) == 2
    # masked layout with K == 0 is not supported
    assert lib.fgg_grouped_gemm_scaled(1, 2, 16, 128, 0, g, g, A, g, g, B4, None, g, g, 128, None) == 2
    # FP4 weight tiling: sizes, N not a multiple of 16, K not a multiple of 128, misaligned output
    nb, ns = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.fgg_pack_fp4_weights_bytes(2, 4096, 7168, ctypes.byref(nb), ctypes.byref(ns)) == 0
    assert nb.value == 2 * 4096 * 3584 and ns.value == 2 * 256 * 14 * 256
    assert lib.fgg_pack_fp4_weights_bytes(1, 32, 384, ctypes.byref(nb), ctypes.byref(ns)) == 0
    assert nb.value == 32 * 192 and ns.value == 2 * 1 * 256
    assert lib.fgg_pack_fp4_weights_bytes(1, 40, 384, ctypes.byref(nb), ctypes.byref(ns)) == 2
    assert lib.fgg_pack_fp4_weights(g, g, 1, 32, 200, g, g, None) == 2
    assert lib.fgg_pack_fp4_weights(g, g, 1, 32, 256, ctypes.c_void_p(g.value + 8), g, None) == 1
    # W4A4 always needs its workspace (the fp16 operand copies)
    nbytes = ctypes.c_size_t(0)
    assert lib.fgg_scaled_gemm_workspace(256, 128, 256, W, W, None, ctypes.byref(nbytes)) == 0
    assert nbytes.value >= 2 * (256 * 256 + 128 * 256)
    assert lib.fgg_scaled_gemm(256, 128, 256, g, g, W, g, g, W, None, g, 128, None, 0, None) == 1
    # W4A4 with K == 0 is not supported
    assert lib.fgg_scaled_gemm(256, 128, 0, g, g, W, g, g, W, None, g, 128, None, 0, None) == 2
    # N % 128 for the FP8 and per-16 W4A4 forms; MXFP4 takes N % 16 but not N % 8
    F8a, F8b = _q(fgg.Q_E4M3_1x128), _q(fgg.Q_E4M3_128x128)
    assert lib.fgg_scaled_gemm(256, 192, 256, g, g, F8a, g, g, F8b, None, g, 192, None, 0, None) == 2
    assert lib.fgg_scaled_gemm(256, 192, 256, g, g, W, g, g, W, None, g, 192, g, 1 << 22, None) == 2
    MX = _q(fgg.Q_E2M1_E8M0_1x32)
    assert lib.fgg_scaled_gemm(256, 200, 256, g, g, MX, g, g, MX, None, g, 200, None, 0, None) == 2
    assert lib.fgg_scaled_gemm(256, 192, 0, g, g, MX, g, g, MX, None, g, 192, None, 0, None) == 2
    # MXFP4: rank 16 is not supported; rank 32 needs its [M][32] workspace
    epi16 = fgg.Epilogue(4096, 4096, 4096, 16, None)
    assert lib.fgg_scaled_gemm(256, 192, 256, g, g, MX, g, g, MX, ctypes.byref(epi16), g, 192, g, 1 << 20, None) == 2
    epi32 = fgg.Epilogue(4096, 4096, 4096, 32, None)
    assert lib.fgg_scaled_gemm_workspace(256, 192, 256, MX, MX, ctypes.byref(epi32), ctypes.byref(nbytes)) == 0
    assert nbytes.value == 256 * 32 * 2
    assert lib.fgg_scaled_gemm(256, 192, 256, g, g, MX, g, g, MX, ctypes.byref(epi32), g, 192, g, 100, None) == 1
    assert lib.fgg_scaled_gemm_workspace(256, 192, 256, MX, MX, None, ctypes.byref(nbytes)) == 0
    assert nbytes.value == 0
    # permute: bad k / E, missing workspace
    assert lib.fgg_moe_permute(g, 10, 0, 4, 128, None, None, 0, g, g, g, g, None, None, 100, g, 1 << 20, None) == 1
    assert lib.fgg_moe_permute(g, 10, 2, 2000, 128, None, None, 0, g, g, g, g, None, None, 100, g, 1 << 20, None) == 1
    assert lib.fgg_moe_permute(g, 10, 2, 4, 128, None, None, 0, g, g, g, g, None, None, 100, None, 0, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.fgg_moe_permute_workspace(10, 2, 4, ctypes.byref(n)) == 0 and n.value > 0
    # fused permute + quantize: bad dtype, K not a multiple of 128, short row stride, missing workspace
    Q = lib.fgg_moe_permute_quantize
    assert Q(g, 10, 2, 4, 128, g, fgg.FGG_E4M3, 256, 256, g, g, g, g, g, g, 100, g, 1 << 20, None) == 2
    assert Q(g, 10, 2, 4, 128, g, fgg.FGG_BF16, 200, 256, g, g, g, g, g, g, 100, g, 1 << 20, None) == 2
    assert Q(g, 10, 2, 4, 128, g, fgg.FGG_BF16, 256, 128, g, g, g, g, g, g, 100, g, 1 << 20, None) == 1
    assert Q(g, 10, 2, 4, 128, g, fgg.FGG_BF16, 256, 256, g, g, g, g, g, g, 100, None, 0, None) == 1
    assert Q(g, 10, 2, 2000, 128, g, fgg.FGG_BF16, 256, 256, g, g, g, g, g, g, 100, g, 1 << 20, None) == 1
    # fused gate-up + SiLU requant: I not a multiple of 128, FP4 weights, missing offsets
    F = lib.fgg_grouped_gemm_silu_quantize
    assert F(2, 256, 100, 256, g, g, A, g, g, B8, g, None, g, g, None) == 2
    assert F(2, 256, 128, 256, g, g, A, g, g, B4, g, None, g, g, None) == 2
    assert F(2, 256, 128, 256, g, g, A, g, g, B8, None, None, g, g, None) == 1
    assert F(0, 256, 128, 256, g, g, A, g, g, B8, g, None, g, g, None) == 1
    # combine: N not a multiple of 8
    assert lib.fgg_moe_combine(g, 16, g, g, 4, 2, 12, g, 16, None) == 2
    # fused down GEMM + combine: workspace size, N not a multiple of 128, missing counts,
    # short workspace, FP4 weights, ldo below N
    n = ctypes.c_size_t(0)
    assert lib.fgg_moe_down_combine_workspace(300, ctypes.byref(n)) == 0 and n.value == 384 * 8
    DC = lib.fgg_moe_down_combine
    assert DC(2, 256, 200, 256, g, g, A, g, g, B8, g, g, g, g, g, 8, 2, g, 200, g, 4096, g, 200, None) == 2
    assert DC(2, 256, 256, 256, g, g, A, g, g, B8, g, None, g, g, g, 8, 2, g, 256, g, 4096, g, 256, None) == 1
    assert DC(2, 256, 256, 256, g, g, A, g, g, B8, g, g, g, g, g, 8, 2, g, 256, g, 1024, g, 256, None) == 1
    assert DC(2, 256, 256, 256, g, g, A, g, g, B4, g, g, g, g, g, 8, 2, g, 256, g, 4096, g, 256, None) == 2
    assert DC(2, 256, 256, 256, g, g, A, g, g, B8, g, g, g, g, g, 8, 2, g, 256, g, 4096, g, 128, None) == 1
