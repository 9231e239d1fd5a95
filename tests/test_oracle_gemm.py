"""Pins for the oracle's GEMMs: the per-group formula against dequantize-then-
matmul and a pure-Python loop, one group against the dense call, closed forms,
scale linearity, the per-tensor special case, and masked vs contiguous."""

import numpy as np
import pytest

import oracle
import synth
from oracle import formats as F


def _quant_problem(seed, M, N, K, G=1, offsets=None):
    g = synth.rng(seed)
    x = synth.normal(g, (M, K))
    w = synth.normal(g, (G, N, K), 0.02)
    aq, sa = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N // 128, K // 128), np.float32)
    for e in range(G):
        bq[e], sb[e] = oracle.quantize_e4m3_blocks(w[e], 128, 128)
    if offsets is None:
        offsets = np.linspace(0, M, G + 1).astype(np.int64)
    return aq, sa, bq, sb, np.asarray(offsets)


def _dequant_a(aq, sa):
    return F.decode_e4m3(aq) * np.repeat(sa.astype(np.float64), 128, axis=1)


def _dequant_b(bq, sb):
    return F.decode_e4m3(bq) * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)


def test_grouped_equals_dequantize_then_matmul():
    # "dequantize, then a plain GEMM" and "scales inside the K loop" compute the same sum
    aq, sa, bq, sb, off = _quant_problem(31, 384, 256, 512, G=3, offsets=[0, 128, 128, 384])
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, off)
    ad = _dequant_a(aq, sa)
    for g in range(3):
        r = slice(off[g], off[g + 1])
        if off[g] == off[g + 1]:
            continue
        ref = ad[r] @ _dequant_b(bq[g], sb[g]).T
        np.testing.assert_allclose(y[r], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_grouped_python_loop_tiny():
    aq, sa, bq, sb, off = _quant_problem(32, 16, 128, 256, G=2, offsets=[0, 7, 16])
    bq, sb = bq[:, :16], sb                 # 16 columns of each expert (one 128-row scale block)
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb[:, :1], off)
    for r in range(16):
        g = 0 if r < 7 else 1
        for n in range(16):
            acc = 0.0
            for kb in range(2):
                part = 0.0
                for kk in range(128):
                    k = kb * 128 + kk
                    part += F.E4M3_TABLE[aq[r, k]] * F.E4M3_TABLE[bq[g, n, k]]
                acc += float(sa[r, kb]) * float(sb[g, 0, kb]) * part
            assert y[r, n] == pytest.approx(acc, rel=1e-13, abs=1e-300)


def test_one_group_equals_dense():
    aq, sa, bq, sb, _ = _quant_problem(33, 256, 256, 384)
    y1 = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, np.array([0, 256]))
    y2 = oracle.scaled_gemm_dense(aq, sa, bq[0], sb[0])
    assert np.array_equal(y1, y2)


def test_constant_operands_closed_form():
    M, N, K = 128, 256, 512
    aq = np.full((M, K), 0x3C, np.uint8)            # 1.5
    bq = np.full((1, N, K), 0xB0, np.uint8)         # -0.5
    sa = np.full((M, K // 128), 0.25, np.float32)
    sb = np.full((1, N // 128, K // 128), 4.0, np.float32)
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, np.array([0, M]))
    assert F.E4M3_TABLE[0xB0] == -0.5
    assert np.all(y == K * 1.5 * -0.5 * 0.25 * 4.0)


def test_power_of_two_scale_linearity():
    aq, sa, bq, sb, off = _quant_problem(34, 256, 128, 256, G=2, offsets=[0, 128, 256])
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, off)
    sa2 = sa.copy()
    sa2[5] *= 2
    sb2 = sb.copy()
    sb2[1] *= 0.5
    y2 = oracle.grouped_gemm_contiguous(aq, sa2, bq, sb2, off)
    assert np.array_equal(y2[5], 2 * y[5])
    assert np.array_equal(y2[128:], 0.5 * y[128:])
    assert np.array_equal(np.delete(y2[:128], 5, 0), np.delete(y[:128], 5, 0))


def test_per_tensor_special_case():
    # scales constant along K and over rows/columns: C·(A_scale·B_scale) of the fp8_gemm sketch
    aq, sa, bq, sb, _ = _quant_problem(35, 128, 256, 384)
    sa[:] = np.float32(0.0123)
    sb[:] = np.float32(3.5)
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, np.array([0, 128]))
    c = F.decode_e4m3(aq) @ F.decode_e4m3(bq[0]).T
    np.testing.assert_allclose(y, c * (float(np.float32(0.0123)) * 3.5), rtol=1e-13)


def test_identity_weights_return_dequantized_rows():
    M, K = 128, 256
    aq, sa, _, _, _ = _quant_problem(36, M, K, K)
    bq = np.zeros((1, K, K), np.uint8)
    bq[0][np.arange(K), np.arange(K)] = 0x38      # 1.0 on the diagonal
    sb = np.ones((1, K // 128, K // 128), np.float32)
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, np.array([0, M]))
    assert np.array_equal(y, _dequant_a(aq, sa))


def test_rows_subset_and_padding_rows():
    aq, sa, bq, sb, off = _quant_problem(37, 384, 128, 256, G=2, offsets=[0, 256, 384])
    aq[200:256] = 0
    sa[200:256] = 0
    y = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, off)
    assert np.all(y[200:256] == 0)
    rows = np.array([3, 255, 300, 383])
    assert np.array_equal(oracle.grouped_gemm_contiguous(aq, sa, bq, sb, off, rows=rows), y[rows])


def test_masked_equals_contiguous_fp8():
    G, Mx, N, K = 3, 16, 128, 256
    masked = np.array([16, 1, 9])
    aq, sa, bq, sb, _ = _quant_problem(38, G * Mx, N, K, G=G)
    y_m = oracle.grouped_gemm_masked(aq.reshape(G, Mx, K), sa.reshape(G, Mx, K // 128), bq, sb,
                                     masked, b_format="e4m3")
    y_c = oracle.grouped_gemm_contiguous(aq, sa, bq, sb, np.arange(G + 1) * Mx)
    for g in range(G):
        assert np.array_equal(y_m[g, :masked[g]], y_c[g * Mx:g * Mx + masked[g]])
        assert np.all(np.isnan(y_m[g, masked[g]:]))


def test_masked_fp4_equals_dequantize_then_matmul():
    g = synth.rng(39)
    G, Mx, N, K = 2, 16, 64, 256
    x = synth.normal(g, (G * Mx, K))
    w = synth.normal(g, (G, N, K), 0.02)
    aq, sa = oracle.quantize_e4m3_blocks(x, 1, 128)
    bcodes = np.empty((G, N, K), np.uint8)
    be = np.empty((G, N, K // 32), np.uint8)
    for e in range(G):
        bcodes[e], be[e] = oracle.quantize_e2m1_e8m0_groups(w[e], 32)
    bp = F.pack_e2m1x2(bcodes)
    masked = np.array([5, 16])
    y = oracle.grouped_gemm_masked(aq.reshape(G, Mx, K), sa.reshape(G, Mx, 2), bp, be, masked)
    ad = _dequant_a(aq, sa).reshape(G, Mx, K)
    for e in range(G):
        bd = F.decode_e2m1(bcodes[e]) * np.repeat(F.decode_e8m0(be[e]), 32, axis=1)
        ref = ad[e, :masked[e]] @ bd.T
        np.testing.assert_allclose(y[e, :masked[e]], ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())
    # one-hot probe: a single nonzero nibble lands on exactly one output column
    bp2 = np.zeros_like(bp)
    bp2[1, 7, 33] = 0x20                      # element k=67 (odd -> high nibble) of column 7 = 1.0
    be2 = np.full_like(be, 127)
    y2 = oracle.grouped_gemm_masked(aq.reshape(G, Mx, K), sa.reshape(G, Mx, 2), bp2, be2, masked)
    expect = F.decode_e4m3(aq.reshape(G, Mx, K)[1, :, 67]) * sa.reshape(G, Mx, 2)[1, :, 0]
    assert np.array_equal(y2[1, :, 7], expect)
    assert np.count_nonzero(y2[1][:, np.arange(N) != 7]) == 0


def test_w4a4_brute_force_and_branches():
    g = synth.rng(40)
    M, N, K, r = 32, 48, 64, 4
    x = synth.to_bf16_values(synth.normal(g, (M, K)))
    w = synth.normal(g, (N, K), 0.02)
    ld = synth.to_bf16_values(synth.normal(g, (K, r), 0.01))
    lu = synth.to_bf16_values(synth.normal(g, (r, N), 0.01))
    b = synth.to_bf16_values(synth.normal(g, (N,), 0.1))
    qx, sx = oracle.quantize_e2m1_fp32_groups(x, 16)
    qw, sw = oracle.quantize_e2m1_fp32_groups(w, 16)
    y = oracle.w4a4_lowrank_gemm(qx, sx, qw, sw, x, ld, lu, b)
    xd = F.decode_e2m1(qx) * np.repeat(sx.astype(np.float64), 16, axis=1)
    wd = F.decode_e2m1(qw) * np.repeat(sw.astype(np.float64), 16, axis=1)
    ref = xd @ wd.T + (x.astype(np.float64) @ ld) @ lu + b
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    # a pure-Python loop on a few entries
    for (i, j) in [(0, 0), (5, 17), (31, 47)]:
        acc = sum(float(F.E2M1_TABLE[qx[i, k]]) * float(F.E2M1_TABLE[qw[j, k]]) * float(sx[i, k // 16]) * float(sw[j, k // 16])
                  for k in range(K))
        acc += sum(float(x[i, k]) * float(ld[k, q]) * float(lu[q, j]) for k in range(K) for q in range(r))
        acc += float(b[j])
        assert y[i, j] == pytest.approx(acc, rel=1e-12, abs=1e-14)
    # the low-rank and bias branches are additive and optional
    y0 = oracle.w4a4_lowrank_gemm(qx, sx, qw, sw)
    np.testing.assert_allclose(y - y0, (x.astype(np.float64) @ ld) @ lu + b, rtol=1e-10, atol=1e-14)


# ------------------------------------------------------------ MXFP4 A4W4

def _mx_problem(seed, M, N, K, r=4):
    g = synth.rng(seed)
    x = synth.to_bf16_values(synth.normal(g, (M, K)))
    w = synth.normal(g, (N, K), 0.02)
    qx, ex = oracle.quantize_e2m1_e8m0_groups(x, 32)
    qw, ew = oracle.quantize_e2m1_e8m0_groups(w, 32)
    ld = synth.to_bf16_values(synth.normal(g, (K, r), 0.01))
    lu = synth.to_bf16_values(synth.normal(g, (r, N), 0.01))
    b = synth.to_bf16_values(synth.normal(g, (N,), 0.1))
    return x, w, qx, ex, qw, ew, ld, lu, b


def test_mxfp4_brute_force_and_python_loop():
    M, N, K, r = 24, 40, 128, 4
    x, w, qx, ex, qw, ew, ld, lu, b = _mx_problem(41, M, N, K, r)
    y = oracle.mxfp4_lowrank_gemm(qx, ex, qw, ew, x, ld, lu, b)
    xd = F.decode_e2m1(qx) * np.repeat(np.ldexp(1.0, ex.astype(int) - 127), 32, axis=1)
    wd = F.decode_e2m1(qw) * np.repeat(np.ldexp(1.0, ew.astype(int) - 127), 32, axis=1)
    np.testing.assert_allclose(y, xd @ wd.T + (x.astype(np.float64) @ ld) @ lu + b, rtol=1e-12, atol=1e-14)
    for (i, j) in [(0, 0), (7, 31), (23, 39)]:
        acc = 0.0
        for k in range(K):
            acc += (float(F.E2M1_TABLE[qx[i, k]]) * 2.0 ** (int(ex[i, k // 32]) - 127)
                    * float(F.E2M1_TABLE[qw[j, k]]) * 2.0 ** (int(ew[j, k // 32]) - 127))
        for k in range(K):
            for q in range(r):
                acc += float(x[i, k]) * float(ld[k, q]) * float(lu[q, j])
        acc += float(b[j])
        assert y[i, j] == pytest.approx(acc, rel=1e-12, abs=1e-14)


def test_mxfp4_equals_w4a4_with_the_same_scales_as_fp32():
    """The MX form is the per-group formula with fp32 scales that happen to be
    powers of two: each E8M0 scale written as an fp32 scale for both 16-element
    halves of its 32-element group gives the same result through the W4A4 oracle
    (an independent loop over 16-element groups)."""
    M, N, K = 16, 24, 256
    x, w, qx, ex, qw, ew, ld, lu, b = _mx_problem(42, M, N, K)
    sx16 = np.repeat(np.ldexp(1.0, ex.astype(int) - 127), 2, axis=1).astype(np.float32)
    sw16 = np.repeat(np.ldexp(1.0, ew.astype(int) - 127), 2, axis=1).astype(np.float32)
    np.testing.assert_allclose(oracle.mxfp4_lowrank_gemm(qx, ex, qw, ew, x, ld, lu, b),
                               oracle.w4a4_lowrank_gemm(qx, sx16, qw, sw16, x, ld, lu, b), rtol=1e-13, atol=1e-15)


def test_mxfp4_closed_form_and_one_hot_scales():
    M, N, K = 8, 8, 128
    # every code 1.5 (E2M1 0x3) against every code -3 (0xD), unit scales: K · 1.5 · -3 exactly
    qx = np.full((M, K), 0x3, np.uint8)
    qw = np.full((N, K), 0xD, np.uint8)
    e1 = np.full((M, K // 32), 127, np.uint8)
    f1 = np.full((N, K // 32), 127, np.uint8)
    assert np.all(oracle.mxfp4_lowrank_gemm(qx, e1, qw, f1) == K * 1.5 * -3.0)
    # one nonzero pair at (m, k) and (n, k): exactly one output, scaled by the two E8M0
    # bytes of k's 32-group (distinct powers of two per row and group identify them)
    ex = (120 + np.arange(M * (K // 32)).reshape(M, K // 32) % 13).astype(np.uint8)
    ew = (125 + np.arange(N * (K // 32)).reshape(N, K // 32) % 7).astype(np.uint8)
    for (m, n, k) in [(0, 0, 0), (3, 5, 33), (7, 7, 127), (2, 6, 64)]:
        a = np.zeros((M, K), np.uint8)
        a[m, k] = 0x2                                  # 1.0
        bw = np.zeros((N, K), np.uint8)
        bw[n, k] = 0xF                                 # -6.0
        y = oracle.mxfp4_lowrank_gemm(a, ex, bw, ew)
        expect = np.zeros((M, N))
        expect[m, n] = -6.0 * 2.0 ** (int(ex[m, k // 32]) - 127) * 2.0 ** (int(ew[n, k // 32]) - 127)
        assert np.array_equal(y, expect), (m, n, k)
    # raising one row's E8M0 exponents by one doubles that row exactly
    x, w, qx, ex, qw, ew, *_ = _mx_problem(43, 12, 16, 256)
    y = oracle.mxfp4_lowrank_gemm(qx, ex, qw, ew)
    ex2 = ex.copy()
    ex2[5] += 1
    y2 = oracle.mxfp4_lowrank_gemm(qx, ex2, qw, ew)
    assert np.array_equal(y2[5], 2 * y[5]) and np.array_equal(np.delete(y2, 5, 0), np.delete(y, 5, 0))


def test_mxfp4_quantized_product_tracks_the_real_product():
    """Both operands quantized with the never-clipping E8M0 rule: the quantized
    product differs from the fp64 product of the unquantized operands by the
    E2M1 rounding only (a few percent of rms), which catches an inverted or
    misplaced scale (that would be off by powers of two)."""
    M, N, K = 64, 64, 512
    x, w, qx, ex, qw, ew, *_ = _mx_problem(44, M, N, K)
    y = oracle.mxfp4_lowrank_gemm(qx, ex, qw, ew)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.sqrt(np.mean((y - ref) ** 2)) < 0.2 * rms
