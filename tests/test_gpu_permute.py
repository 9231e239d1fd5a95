"""GPU parity: moe_permute (bit-exact indices, rows and scales) and
moe_combine (tolerance; exact for the one-slot unit-weight gather)."""

import os

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from _util import cuda, to_np, tol_check

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_permute(ids, E, align=128, K=256, seed=0, m_cap=None):
    T, k = ids.shape
    g = synth.rng(seed)
    xq = g.integers(0, 256, size=(T, K), dtype=np.uint8)
    xs = g.random((K // 128, T), dtype=np.float32) + np.float32(0.5)       # device layout [K/128, T]
    got = fgg.moe_permute(cuda(ids), E, align, xq=cuda(xq), xs=cuda(xs), m_cap=m_cap)
    ref = oracle.moe_permute(ids, E, align)
    mt = int(ref["offsets"][-1])
    assert np.array_equal(to_np(got["offsets"]), ref["offsets"])
    assert np.array_equal(to_np(got["counts"]), ref["counts"])
    assert np.array_equal(to_np(got["src_to_row"]), ref["src_to_row"])
    m_cap = got["m_cap"]
    assert np.array_equal(to_np(got["row_to_src"]), ref["row_to_src"][:m_cap])
    a_ref, sa_ref = oracle.gather_permuted(ref["row_to_src"], mt, k, xq, xs.T)
    assert np.array_equal(to_np(got["a"])[:mt], a_ref)
    assert np.array_equal(to_np(got["sa"])[:, :mt], sa_ref.T)
    return got, ref


def test_permute_two_experts_eight_tokens():
    d = {}
    for line in open(os.path.join(GOLDEN, "permute_2x8.txt")):
        line = line.split("#")[0].strip()
        if line:
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    ids = np.array(d["topk_ids"], dtype=np.int32).reshape(d["T"][0], d["k"][0])
    got, _ = _check_permute(ids, 2)
    assert to_np(got["src_to_row"]).tolist() == d["src_to_row"]


def test_permute_tiny_moe_routing():
    w = synth.tiny_moe()
    _check_permute(w["topk_ids"], 4, K=256, seed=1)


@pytest.mark.parametrize("T,k,E,align", [(1, 1, 1, 128), (300, 8, 32, 128), (1000, 6, 17, 128),
                                         (5000, 4, 256, 128), (777, 3, 5, 16), (70000, 2, 1024, 128)])
def test_permute_random_with_dropped_ids(T, k, E, align):
    g = synth.rng(T + k + E)
    ids = g.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    _check_permute(ids, E, align, K=128, seed=2)


def test_permute_all_dropped_and_one_expert():
    ids = np.full((64, 4), -1, np.int32)
    got, ref = _check_permute(ids, 8)
    assert ref["offsets"][-1] == 0
    ids = np.zeros((64, 4), np.int32)                    # everything to expert 0
    _check_permute(ids, 8)


def test_permute_moe_prefill_routing_full_size():
    ids = synth.moe_prefill_routing()["topk_ids"]
    got, ref = _check_permute(ids, 32, K=7168, seed=3)
    assert int(ref["offsets"][-1]) == 10112


def test_permute_small_m_cap_writes_nothing_beyond():
    ids = np.zeros((64, 2), np.int32)                    # needs 128 rows
    g = synth.rng(9)
    xq = cuda(g.integers(0, 256, size=(64, 128), dtype=np.uint8))
    xs = cuda(np.ones((1, 64), np.float32))
    got = fgg.moe_permute(cuda(ids), 2, 128, xq=xq, xs=xs, m_cap=100)
    assert to_np(got["offsets"]).tolist() == [0, 128, 128]      # the true total is still reported
    r2s = to_np(got["row_to_src"])
    assert r2s.shape == (100,) and np.array_equal(r2s, np.arange(100))


def test_permute_zero_tokens():
    ids = np.zeros((0, 4), np.int32)
    got = fgg.moe_permute(cuda(ids), 3, 128)
    assert to_np(got["offsets"]).tolist() == [0, 0, 0, 0]
    assert to_np(got["counts"]).tolist() == [0, 0, 0]


@pytest.mark.parametrize("T,k,E,N", [(64, 2, 4, 512), (8192, 8, 32, 7168), (33, 3, 5, 8)])
def test_combine(T, k, E, N):
    g = synth.rng(T * 7 + N)
    ids = g.integers(-1, E, size=(T, k)).astype(np.int32)
    ref_perm = oracle.moe_permute(ids, E, 128)
    mt = int(ref_perm["offsets"][-1])
    y = synth.to_bf16_values(synth.normal(g, (max(mt, 1), N)))
    w = g.random((T, k)).astype(np.float32)
    out = fgg.moe_combine(cuda(y, torch.bfloat16), cuda(ref_perm["src_to_row"]), cuda(w))
    ref = oracle.round_bf16(oracle.moe_combine(y, ref_perm["src_to_row"], w, T, k))
    tol_check(to_np(out), ref, what="combine")
    none = np.all(ids < 0, axis=1)
    assert np.all(to_np(out)[none] == 0)


def test_combine_unit_weight_single_slot_is_exact_gather():
    g = synth.rng(77)
    T, E, N = 500, 6, 1024
    ids = g.integers(0, E, size=(T, 1)).astype(np.int32)
    ref_perm = oracle.moe_permute(ids, E, 128)
    y = synth.to_bf16_values(synth.normal(g, (int(ref_perm["offsets"][-1]), N)))
    out = fgg.moe_combine(cuda(y, torch.bfloat16), cuda(ref_perm["src_to_row"]), cuda(np.ones((T, 1), np.float32)))
    assert np.array_equal(to_np(out), y[ref_perm["src_to_row"]])


# ------------------------------------------------ fused quantize + permute

def _x_input(seed, T, K, dtype):
    x = synth.normal(synth.rng(seed), (T, K)) * np.float32(2.0)
    if T > 3:
        x[1, :128] = 0.0                  # an all-zero group
        x[2, 5] = 1e30                    # one huge value sets its group's scale
        x[3, 7] = -0.0                    # signed zero keeps its sign code
        x[3, 130:140] = 1e-30             # tiny values beside normal ones
    if dtype == torch.bfloat16:
        x = synth.to_bf16_values(x)
    return x


@pytest.mark.parametrize("T,k,E,K,dtype", [(64, 2, 4, 256, torch.bfloat16), (300, 8, 32, 640, torch.float32),
                                           (1000, 6, 17, 1152, torch.bfloat16), (5000, 4, 256, 128, torch.float32),
                                           (777, 3, 5, 2560, torch.bfloat16)])
def test_permute_quantize_matches_oracle_and_unfused(T, k, E, K, dtype):
    g = synth.rng(T + 3 * k + E + K)
    ids = g.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    x = _x_input(T + K, T, K, dtype)
    xt = cuda(x, dtype)
    out = fgg.moe_permute_outputs(T, k, E, 128, K)
    out["a"].fill_(0xAB)
    out["sa"].fill_(-7.0)
    got = fgg.moe_permute(cuda(ids), E, 128, x=xt, out=out)
    ref = oracle.moe_permute(ids, E, 128)
    mt = int(ref["offsets"][-1])
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    a_ref, s_ref = oracle.gather_permuted(ref["row_to_src"], mt, k, aq_r, sa_r)
    assert np.array_equal(to_np(got["offsets"]), ref["offsets"])
    assert np.array_equal(to_np(got["src_to_row"]), ref["src_to_row"])
    assert np.array_equal(to_np(got["row_to_src"]), ref["row_to_src"][:got["m_cap"]])
    a, sa = to_np(got["a"]), to_np(got["sa"])
    assert np.array_equal(a[:mt], a_ref)
    assert np.array_equal(sa[:, :mt], s_ref.T)
    assert np.all(a[mt:] == 0xAB) and np.all(sa[:, mt:] == -7.0)       # rows >= M_total untouched
    # the unfused pair of calls gives the same bytes
    xq, xs = fgg.quantize_blockwise(xt, fgg.Q_E4M3_1x128)
    unf = fgg.moe_permute(cuda(ids), E, 128, xq=xq, xs=xs)
    assert torch.equal(unf["a"][:mt], got["a"][:mt]) and torch.equal(unf["sa"][:, :mt], got["sa"][:, :mt])


def test_permute_quantize_moe_prefill_full_size():
    r = synth.moe_prefill_routing()
    x = synth.to_bf16_values(synth.moe_prefill_x())
    T, K = x.shape
    got = fgg.moe_permute(cuda(r["topk_ids"]), 32, 128, x=cuda(x, torch.bfloat16))
    ref = oracle.moe_permute(r["topk_ids"], 32, 128)
    mt = int(ref["offsets"][-1])
    assert mt == 10112 and np.array_equal(to_np(got["offsets"]), ref["offsets"])
    # sampled rows: each row's codes/scales against the oracle's quantization of its token
    rows = np.array([0, 1, 127, 128, 2323, 2400, 5000, 9000, 10111])
    r2s = ref["row_to_src"][rows]
    a, sa = to_np(got["a"]), to_np(got["sa"])
    for row, p in zip(rows, r2s):
        if p < 0:
            assert np.all(a[row] == 0) and np.all(sa[:, row] == 0)
        else:
            qr, sr = oracle.quantize_e4m3_blocks(x[p // 8][None], 1, 128)
            assert np.array_equal(a[row], qr[0]) and np.array_equal(sa[:, row], sr[0])


def test_permute_quantize_small_m_cap_and_zero_tokens():
    ids = np.zeros((64, 2), np.int32)                    # needs 128 rows
    x = cuda(_x_input(5, 64, 128, torch.float32))
    out = fgg.moe_permute_outputs(64, 2, 2, 128, 128, m_cap=100)
    got = fgg.moe_permute(cuda(ids), 2, 128, x=x, out=out)
    assert to_np(got["offsets"]).tolist() == [0, 128, 128]
    assert np.array_equal(to_np(got["row_to_src"]), np.arange(100))
    aq_r, sa_r = oracle.quantize_e4m3_blocks(to_np(x), 1, 128)
    a = to_np(got["a"])
    assert np.array_equal(a[:100], aq_r[np.arange(100) // 2])
    got0 = fgg.moe_permute(cuda(np.zeros((0, 4), np.int32)), 3, 128, x=torch.zeros((0, 256), device="cuda"))
    assert to_np(got0["offsets"]).tolist() == [0, 0, 0, 0]


def test_undersized_m_cap_nothing_beyond_it():
    """M_cap smaller than the routed rows need: pairs whose row would be at or past
    M_cap are reported as dropped (src_to_row = -1), the grouped GEMMs called with
    M = M_cap stop at row M_cap (guard rows after the output stay untouched), and the
    combine of those outputs is the oracle's combine without the dropped pairs."""
    T, k, E, K, N, I = 200, 2, 3, 256, 256, 128
    g = synth.rng(55)
    ids = g.integers(0, E, size=(T, k)).astype(np.int32)
    ref = oracle.moe_permute(ids, E, 128)
    offsets = ref["offsets"]
    m_cap = int(offsets[1]) + 50                  # inside expert 1's segment; expert 2 lies beyond
    assert m_cap < int(offsets[-1]) - 128
    x = synth.normal(g, (T, K))
    out = fgg.moe_permute_outputs(T, k, E, 128, K, m_cap=m_cap)
    perm = fgg.moe_permute(cuda(ids), E, 128, x=cuda(x), out=out)
    s2r = ref["src_to_row"].copy()
    s2r[s2r >= m_cap] = -1
    assert np.array_equal(to_np(perm["offsets"]), offsets)            # the true total is still reported
    assert np.array_equal(to_np(perm["src_to_row"]), s2r)
    assert np.array_equal(to_np(perm["row_to_src"]), ref["row_to_src"][:m_cap])
    w = synth.normal(g, (E, N, K), 0.02)
    bq = torch.stack([fgg.quantize_blockwise(cuda(w[e]), fgg.Q_E4M3_128x128)[0] for e in range(E)])
    sb = torch.stack([fgg.quantize_blockwise(cuda(w[e]), fgg.Q_E4M3_128x128)[1] for e in range(E)])
    guard = torch.full((m_cap + 64, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(perm["a"], perm["sa"], bq, sb, offsets=perm["offsets"], out=guard[:m_cap])
    y = to_np(guard)
    assert np.all(np.isnan(y[m_cap:]))
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    a_r, s_r = oracle.gather_permuted(ref["row_to_src"], int(offsets[-1]), k, aq_r, sa_r)
    bq_r = np.stack([oracle.quantize_e4m3_blocks(w[e], 128, 128)[0] for e in range(E)])
    sb_r = np.stack([oracle.quantize_e4m3_blocks(w[e], 128, 128)[1] for e in range(E)])
    y_ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(a_r, s_r, bq_r, sb_r, offsets, rows=np.arange(m_cap)))
    tol_check(y[:m_cap], y_ref, what="grouped GEMM with M = M_cap")
    # the SiLU requant instance: codes and scales stop at row M_cap too
    wgu = synth.normal(g, (E, 2 * I, K), 0.02)
    bq2 = torch.stack([fgg.quantize_blockwise(cuda(wgu[e]), fgg.Q_E4M3_128x128)[0] for e in range(E)])
    sb2 = torch.stack([fgg.quantize_blockwise(cuda(wgu[e]), fgg.Q_E4M3_128x128)[1] for e in range(E)])
    qg = torch.full((m_cap + 64, I), 0xAB, dtype=torch.uint8, device="cuda")
    sg = torch.full(((I // 128) * m_cap + 64,), -3.0, dtype=torch.float32, device="cuda")
    fgg.grouped_gemm_silu_quantize(perm["a"], perm["sa"], bq2, sb2, perm["offsets"], out=qg[:m_cap],
                                   scales=sg[:(I // 128) * m_cap].view(I // 128, m_cap))
    assert np.all(to_np(qg)[m_cap:] == 0xAB) and np.all(to_np(sg)[(I // 128) * m_cap:] == -3.0)
    # combine over the GEMM output of M_cap rows
    tw = g.random((T, k)).astype(np.float32)
    got = fgg.moe_combine(guard[:m_cap], perm["src_to_row"], cuda(tw))
    ref_out = oracle.round_bf16(oracle.moe_combine(y_ref, s2r, tw, T, k))
    tol_check(to_np(got), ref_out, what="combine with dropped pairs past M_cap")
