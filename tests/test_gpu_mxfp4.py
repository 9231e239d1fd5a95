"""GPU parity of the MXFP4 W4A4 path (fgg_scaled_gemm with E2M1 + E8M0 per 32 on
both operands, optional rank-32 low-rank branch and bias) against the oracle's
mxfp4_lowrank_gemm, every output: one-hot probes that pin both operands' FP4
lane layout, nibble order and the placement of each per-32 E8M0 scale, small and
partial-tile shapes, and the full 4096 x 3072 x 3072 shape.

Tolerance: |y - y_ref| <= 1e-2 · (|y_ref| + rms(y_ref)).  Every FP4 product and
its power-of-two scaling is exact, so the GPU's error is the matrix core's block
sums (~1e-4 of the sum of |products|, measured), the bf16 rounding of the
low-rank intermediate T, and the bf16 output rounding."""

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from oracle import formats as F
from _util import cuda, pmap, to_np, tol_check

pytestmark = pytest.mark.gpu


def test_one_hot_probe_mxfp4():
    """A single 1.0 at (m, k) of A and -6 at (n, k) of B give exactly one output,
    (m, n) = -6 · 2^(ea[m, k/32] - 127) · 2^(eb[n, k/32] - 127): pins the FP4
    operand layout of both operands, the nibble order and which lane's E8M0 byte
    scales which 32 K elements."""
    M, N, K = 256, 192, 256
    ea = (118 + np.arange(M * (K // 32)).reshape(M, K // 32) % 17).astype(np.uint8)
    eb = (121 + np.arange(N * (K // 32)).reshape(N, K // 32) % 11).astype(np.uint8)
    for (m, n, k) in [(0, 0, 0), (255, 191, 255), (17, 5, 33), (130, 64, 96), (3, 100, 127), (200, 150, 128),
                      (64, 31, 63), (1, 2, 190)]:
        a = np.zeros((M, K // 2), np.uint8)
        a[m, k // 2] = 0x2 << (4 * (k % 2))
        b = np.zeros((N, K // 2), np.uint8)
        b[n, k // 2] = 0xF << (4 * (k % 2))
        y = to_np(fgg.scaled_gemm(cuda(a), cuda(ea), cuda(b), cuda(eb), qdesc="mxfp4"))
        expect = np.zeros((M, N))
        expect[m, n] = -6.0 * 2.0 ** (int(ea[m, k // 32]) - 127) * 2.0 ** (int(eb[n, k // 32]) - 127)
        assert np.array_equal(y, expect), (m, n, k)


def _mx_run(wl, epilogue=True):
    M, N, K = wl["M"], wl["N"], wl["K"]
    xq, xe = fgg.quantize_blockwise(cuda(wl["x"]), fgg.Q_E2M1_E8M0_1x32)
    wq, we = fgg.quantize_blockwise(cuda(wl["w"]), fgg.Q_E2M1_E8M0_1x32)
    kw = {}
    if epilogue:
        kw = dict(x_bf16=cuda(wl["x"], torch.bfloat16), l_down=cuda(wl["l_down"], torch.bfloat16),
                  l_up=cuda(wl["l_up"], torch.bfloat16), bias=cuda(wl["bias"], torch.bfloat16))
    d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.scaled_gemm(xq, xe, wq, we, qdesc="mxfp4", out=d, **kw)
    qx_r, ex_r = oracle.quantize_e2m1_e8m0_groups(wl["x"], 32)
    qw_r, ew_r = oracle.quantize_e2m1_e8m0_groups(wl["w"], 32)
    assert np.array_equal(to_np(xq), F.pack_e2m1x2(qx_r)) and np.array_equal(to_np(xe), ex_r)
    assert np.array_equal(to_np(wq), F.pack_e2m1x2(qw_r)) and np.array_equal(to_np(we), ew_r)
    blocks = [slice(r, r + 256) for r in range(0, M, 256)]
    if epilogue:
        fn = lambda b: oracle.mxfp4_lowrank_gemm(qx_r[b], ex_r[b], qw_r, ew_r, wl["x"][b], wl["l_down"],  # noqa
                                                 wl["l_up"], wl["bias"])
    else:
        fn = lambda b: oracle.mxfp4_lowrank_gemm(qx_r[b], ex_r[b], qw_r, ew_r)  # noqa: E731
    return to_np(d), oracle.round_bf16(np.concatenate(pmap(fn, blocks)))


@pytest.mark.parametrize("M,N,K,epi", [(256, 192, 128, False), (512, 384, 512, True), (300, 208, 384, True),
                                       (1, 16, 128, True), (777, 1008, 640, True), (256, 192, 1024, False)])
def test_mxfp4_small_and_partial_tiles(M, N, K, epi):
    wl = synth.w4a4(seed=81 + M + N, M=M, N=N, K=K)
    y, ref = _mx_run(wl, epilogue=epi)
    tol_check(y, ref, what=f"mxfp4 {M}x{N}x{K}")


def test_mxfp4_lowrank_branch_alone():
    """All-zero codes: the block-scaled product vanishes and the output is the
    low-rank term plus the bias, so that branch is checked without the (much
    larger) main product around it."""
    M, N, K = 256, 384, 768
    wl = synth.w4a4(seed=93, M=M, N=N, K=K)
    ld = synth.to_bf16_values(wl["l_down"] * np.float32(20.0))
    zq = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    ze = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    we = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
    y = fgg.scaled_gemm(zq, ze, wq, we, qdesc="mxfp4", x_bf16=cuda(wl["x"], torch.bfloat16),
                        l_down=cuda(ld, torch.bfloat16), l_up=cuda(wl["l_up"], torch.bfloat16),
                        bias=cuda(wl["bias"], torch.bfloat16))
    ref = oracle.round_bf16(oracle.mxfp4_lowrank_gemm(
        np.zeros((M, K), np.uint8), np.full((M, K // 32), 127, np.uint8), np.zeros((N, K), np.uint8),
        np.full((N, K // 32), 127, np.uint8), wl["x"], ld, wl["l_up"], wl["bias"]))
    assert np.abs(ref).max() > 0.1
    tol_check(to_np(y), ref, what="mxfp4 low-rank branch")


def test_mxfp4_full_size_every_output():
    wl = synth.w4a4()
    y, ref = _mx_run(wl)
    tol_check(y, ref, what="mxfp4 4096x3072x3072 + rank 32 + bias, every output")


def test_mxfp4_deterministic():
    wl = synth.w4a4(seed=97, M=1024, N=768, K=1024)
    xq, xe = fgg.quantize_blockwise(cuda(wl["x"]), fgg.Q_E2M1_E8M0_1x32)
    wq, we = fgg.quantize_blockwise(cuda(wl["w"]), fgg.Q_E2M1_E8M0_1x32)
    kw = dict(x_bf16=cuda(wl["x"], torch.bfloat16), l_down=cuda(wl["l_down"], torch.bfloat16),
              l_up=cuda(wl["l_up"], torch.bfloat16), bias=cuda(wl["bias"], torch.bfloat16))
    y1 = fgg.scaled_gemm(xq, xe, wq, we, qdesc="mxfp4", **kw)
    y2 = fgg.scaled_gemm(xq, xe, wq, we, qdesc="mxfp4", **kw)
    assert torch.equal(y1, y2)


def test_mxfp4_outlier_activations_need_no_fp16_range():
    """Outlier groups far beyond fp16's range (amax 1e6) and tiny ones (1e-6): the
    E8M0 scales span 2^-127..2^127, so the MX path computes them as it does unit
    values."""
    M, N, K = 256, 192, 256
    wl = synth.w4a4(seed=95, M=M, N=N, K=K)
    x = wl["x"].copy()
    x[7, :64] *= np.float32(1e6)
    x[9, 128:160] *= np.float32(1e-6)
    wl = dict(wl, x=synth.to_bf16_values(x))
    y, ref = _mx_run(wl, epilogue=False)
    assert np.all(np.isfinite(y))
    # each row against its own scale (the outlier row's magnitude would swamp a shared rms)
    for r in (7, 9):
        tol_check(y[r], ref[r], what=f"mxfp4 outlier row {r}")
    rest = np.setdiff1d(np.arange(M), [7])
    tol_check(y[rest], ref[rest], what="mxfp4 rows beside the outlier row")
