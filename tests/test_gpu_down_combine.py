"""GPU tests of fgg_moe_down_combine (the down GEMM with the combine of single-slot
tokens in its epilogue): its output equals the two calls it replaces,
fgg_grouped_gemm_scaled (with the permute's counts) then fgg_moe_combine, bit for bit,
and the oracle's combined output within the GEMM tolerance.  Routings mix tokens with
zero, one and several routed slots (ids >= E are dropped); the multi-tile case forces
several persistent tiles per workgroup (the routing table alternates between two LDS
buffers from tile to tile); the full-size case is the prefill step's down projection."""

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from _util import cuda, to_np, tol_check

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F81      # a bf16 NaN pattern no GEMM output has


def _routing(seed, T, k, E, dropped):
    """Per token k distinct ids out of E local + `dropped` non-local ones (dropped)."""
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(E + dropped)[:k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    return ids, w


def _case(seed, T, k, E, dropped, N, K):
    g = np.random.default_rng(seed + 1)
    ids, tw = _routing(seed, T, k, E, dropped)
    x = g.standard_normal((T, K)).astype(np.float32)
    wt = (0.02 * g.standard_normal((E, N, K))).astype(np.float32)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    perm = fgg.moe_permute(cuda(ids), E, 128, xq=xq, xs=xs)
    bq = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        fgg.quantize_blockwise(cuda(wt[e]), fgg.Q_E4M3_128x128, out=bq[e], scales=bs[e])
    return dict(ids=ids, tw=tw, x=x, wt=wt, perm=perm, bq=bq, bs=bs, twd=cuda(tw))


def _two_calls(c):
    p = c["perm"]
    y = fgg.grouped_gemm_scaled(p["a"], p["sa"], c["bq"], c["bs"], offsets=p["offsets"], masked_m=p["counts"])
    out = fgg.moe_combine(y, p["src_to_row"], c["twd"])
    return y, out


def _fused(c):
    p = c["perm"]
    M = p["a"].shape[0]
    N = c["bq"].shape[1]
    y = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = fgg.moe_down_combine(p["a"], p["sa"], c["bq"], c["bs"], p["offsets"], p["counts"], p["src_to_row"],
                               p["row_to_src"], c["twd"], y)
    return y, out


def _check_against_two_calls(c):
    y1, out1 = _two_calls(c)
    y2, out2 = _fused(c)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "fused output differs from the two calls"
    # y: rows of tokens with two or more routed slots equal, rows of single-slot tokens untouched
    s2r = to_np(c["perm"]["src_to_row"]).reshape(len(c["tw"]), -1)
    routed = (s2r >= 0).sum(1)
    multi_rows = s2r[routed >= 2][s2r[routed >= 2] >= 0]
    single_rows = s2r[routed == 1][s2r[routed == 1] >= 0]
    y1i, y2i = to_np(y1.view(torch.int16)), to_np(y2.view(torch.int16))
    assert np.array_equal(y1i[multi_rows], y2i[multi_rows])
    assert (y2i[single_rows] == np.int16(SENTINEL)).all()
    return out2, routed


def _oracle_out(c, T, k, E):
    aq_r, sa_r = oracle.quantize_e4m3_blocks(c["x"], 1, 128)
    p = oracle.moe_permute(c["ids"], E, 128)
    mt = int(p["offsets"][-1])
    a_r, s_r = oracle.gather_permuted(p["row_to_src"], mt, k, aq_r, sa_r)
    G, N, K = c["wt"].shape
    bq_r = np.empty((G, N, K), np.uint8)
    sb_r = np.empty((G, N // 128, K // 128), np.float32)
    for e in range(G):
        bq_r[e], sb_r[e] = oracle.quantize_e4m3_blocks(c["wt"][e], 128, 128)
    y_r = oracle.round_bf16(oracle.grouped_gemm_contiguous(a_r, s_r, bq_r, sb_r, p["offsets"]))
    return oracle.round_bf16(oracle.moe_combine(y_r, p["src_to_row"], c["tw"], T, k))


@pytest.mark.parametrize("T,k,E,dropped,N,K", [(200, 3, 4, 3, 384, 384), (37, 2, 3, 2, 256, 128), (1, 4, 2, 3, 128, 256)])
def test_down_combine_small(T, k, E, dropped, N, K):
    c = _case(11 + T, T, k, E, dropped, N, K)
    out, routed = _check_against_two_calls(c)
    if T > 1:
        assert (routed == 0).any() and (routed == 1).any() and (routed >= 2).any(), "routing lacks a slot mix"
    tol_check(to_np(out), _oracle_out(c, T, k, E), what="fused down + combine")


def test_down_combine_persistent_multi_tile():
    """A grid for 8 CUs (64 workgroups) and ~190 tiles: every workgroup runs several."""
    T, k, E, dropped, N, K = 1600, 3, 8, 2, 1792, 256
    c = _case(5, T, k, E, dropped, N, K)
    fgg.set_num_cus(8)
    try:
        out, _ = _check_against_two_calls(c)
    finally:
        fgg.set_num_cus(0)
    m_tiles = (int(to_np(c["perm"]["offsets"])[-1]) + 127) // 128
    assert m_tiles * (N // 256) > 3 * 64, "fewer than three tiles per workgroup"
    tol_check(to_np(out), _oracle_out(c, T, k, E), what="fused down + combine, multi-tile")


def test_down_combine_prefill_full_size_equals_two_calls():
    import bench
    st = bench.setup_prefill(fgg, synth, torch)
    b, p = st["bufs"], st["perm"]
    bench.prefill_step(fgg, st)          # permute, gate-up: the down GEMM's inputs
    c = dict(perm=dict(a=b["a2"], sa=b["s2"], offsets=p["offsets"], counts=p["counts"],
                       src_to_row=p["src_to_row"], row_to_src=p["row_to_src"]),
             bq=st["dn_q"], bs=st["dn_s"], twd=st["tw"], tw=to_np(st["tw"]))
    _, routed = _check_against_two_calls(c)
    assert (routed == 1).sum() > 1000 and (routed >= 2).sum() > 1000
