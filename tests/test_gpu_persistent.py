"""GPU parity of the grouped GEMMs' persistent multi-tile path on every output.

With the grid forced small (fgg_set_num_cus(8): 64 workgroups) each workgroup
runs several tiles in sequence, so the tile loop, the next tile's stage DMA
issued behind the SiLU epilogue, the LDS ring's reuse across tiles and the
hand-counted vmcnt waits are exercised at sizes the oracle checks in full.
Segment lengths are ragged (empty experts, 1-row and partial tiles, several
M-tiles per expert) and K spans 3 and 7 K blocks (ring wrap-around inside the
unrolled K loop)."""

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from _util import cuda, to_np, tol_check
from test_gpu_gemm import _contig_case, _quant_weights_gpu, _quant_weights_oracle, _silu_requant_close, _valid_rows

pytestmark = pytest.mark.gpu

COUNTS = [300, 0, 129, 640, 1, 255, 70]           # 384+0+256+640+128+256+128 = 1792 rows: 14 M-tiles


@pytest.fixture
def small_grid():
    def set_(n):
        fgg.set_num_cus(n)
    yield set_
    fgg.set_num_cus(0)


def _tile_count(offsets, n_tiles):
    return (int(offsets[-1]) + 127) // 128 * n_tiles


@pytest.mark.parametrize("num_cus,N,K,use_counts", [(8, 3840, 384, False), (8, 3840, 384, True),
                                                      (72, 2048, 896, False), (8, 1920, 896, True)])
def test_grouped_persistent_every_output(small_grid, num_cus, N, K, use_counts):
    x, w, offsets = _contig_case(1000 + N + K, COUNTS, N, K)
    # 64 workgroups (72 CUs: 72) take 210 / 112 / 112 tiles: several per workgroup
    assert _tile_count(offsets, (N + 255) // 256) >= 100
    small_grid(num_cus)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    M = x.shape[0]
    d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    counts = cuda(np.array(COUNTS, np.int32)) if use_counts else None
    fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets), masked_m=counts, out=d)
    y = to_np(d)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = _quant_weights_oracle(w)
    assert np.array_equal(to_np(xq), aq_r) and np.array_equal(to_np(bq), bq_r)
    mt = int(offsets[-1])
    ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(aq_r, sa_r, bq_r, sb_r, offsets))[:mt]
    rows = _valid_rows(offsets, COUNTS) if use_counts else np.arange(mt)
    tol_check(y[rows], ref[rows], what=f"persistent grouped GEMM, grid for {num_cus} CUs")
    rest = np.setdiff1d(np.arange(M), rows)
    if use_counts:
        assert np.all(np.isnan(y[rest]))                        # padding rows not written
    else:
        assert np.all(np.isnan(y[mt:]))
        for e in range(len(COUNTS)):                            # padding rows computed as +0
            pad = y[offsets[e] + COUNTS[e]:offsets[e + 1]]
            assert np.all(pad == 0) and not np.any(np.signbit(pad))
    # the same call on the full grid gives the same bits
    small_grid(0)
    d2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets), masked_m=counts, out=d2)
    assert np.array_equal(to_np(d2)[rows], y[rows])


@pytest.mark.parametrize("num_cus,I,K,use_counts", [(8, 1920, 384, False), (8, 1920, 384, True),
                                                      (72, 1024, 896, True)])
def test_grouped_silu_persistent_every_output(small_grid, num_cus, I, K, use_counts):
    x, w, offsets = _contig_case(2000 + I + K, COUNTS, 2 * I, K)
    small_grid(num_cus)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    M = x.shape[0]
    q = torch.full((M, I), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((I // 128, M), -3.0, dtype=torch.float32, device="cuda")
    counts = cuda(np.array(COUNTS, np.int32)) if use_counts else None
    fgg.grouped_gemm_silu_quantize(xq, xs, bq, sb, cuda(offsets), counts=counts, out=q, scales=s)
    q, s = to_np(q), to_np(s)
    mt = int(offsets[-1])
    rows = _valid_rows(offsets, COUNTS) if use_counts else np.arange(mt)
    rest = np.setdiff1d(np.arange(M), rows)
    assert np.all(q[rest] == 0xAB) and np.all(s[:, rest] == -3.0)
    # the same call on the full grid (each workgroup one or two tiles) gives the same bits
    small_grid(0)
    q2, s2 = fgg.grouped_gemm_silu_quantize(xq, xs, bq, sb, cuda(offsets), counts=counts)
    assert np.array_equal(to_np(q2)[rows], q[rows]) and np.array_equal(to_np(s2)[:, rows], s[:, rows])
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = _quant_weights_oracle(w)
    h = oracle.grouped_gemm_contiguous(aq_r, sa_r, bq_r, sb_r, offsets, rows=rows)   # fp64, not rounded
    q_r, s_r = oracle.silu_mul_quantize(h)
    _silu_requant_close(q[rows], s[:, rows].T, q_r, s_r, h, f"persistent SiLU requant, grid for {num_cus} CUs")


def test_dense_persistent_small_grid_every_output(small_grid):
    """The dense kernel with a 64-workgroup grid: 8 x 9 tiles of 256 x 256 (partial
    last row tile), so some workgroups run two, 7 K blocks."""
    M, N, K = 2000, 2304, 896
    g = synth.rng(4321)
    x = synth.normal(g, (M, K))
    w = synth.normal(g, (N, K), 0.02)
    small_grid(8)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = fgg.quantize_blockwise(cuda(w), fgg.Q_E4M3_128x128)
    y = to_np(fgg.scaled_gemm(xq, xs, bq, sb))
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = oracle.quantize_e4m3_blocks(w, 128, 128)
    tol_check(y, oracle.round_bf16(oracle.scaled_gemm_dense(aq_r, sa_r, bq_r, sb_r)), what="dense, small grid")
