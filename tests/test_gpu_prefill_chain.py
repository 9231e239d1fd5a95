"""The benched prefill MoE step, every output against the oracle layer.

bench.prefill_step is run as timed (fused permute-quantize, gate-up GEMM with
the SiLU(gate)·up e4m3 requantization fused into its epilogue, down GEMM,
combine; both GEMMs given the permute's counts) on the full prefill shape:
8192 tokens, hidden 7168, 32 local experts of 256, top-8, Zipf(1.1) segments.
The weights come from the seeded numpy generators, so the oracle quantizes the
same fp32 values; every stage is compared on every routed row:

  permute    offsets, counts, src_to_row, row_to_src, codes and scales: bit-exact
  weights    e4m3 codes and 128x128 scales of all 64 weight matrices: bit-exact
  gate-up    requantized codes and scales of SiLU(gate)·up, decided on the GPU from
             its fp32 block sums and in the oracle from exact sums.  The matrix
             core's sum of a block's 128 products is accurate to ~1e-4 of the sum
             of their magnitudes (measured: up to 1.6e-4 for codes over the whole
             e4m3 range, 5e-5 for codes in its upper binades), so a GPU quotient
             a/s drifts by up to ~0.0064 code units (measured on this layer) and
             several codes are correct.  Bar: scales within 2e-4 relative; every
             GPU code is the e4m3 rounding of a value within 0.032 code units (5x
             that drift) of the oracle's quotient, i.e. lies between
             enc(q - 0.032) and enc(q + 0.032).
  down       y against the oracle's y (the oracle's own codes): within
             1e-2·(|y_ref| + rms) plus the largest change the validated
             differences of the GPU's inputs can make,
             Σ_k |dq_gpu·s_gpu - dq_ref·s_ref|[r,k] · |B[n,k]|·s_B
  combine    out within 1e-2·(|out_ref| + rms) plus Σ_j w_j·(2^-8·|y_ref_j| + that
             allowance of slot j) (each slot's bf16 rounding and input choices)
The expected values are the oracle's alone; the GPU's codes enter only the
allowance, after the check that they are valid alternatives.  Padding rows of
the down output are not written (counts given)."""

import numpy as np
import pytest
import torch

import bench
import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from oracle import formats as F
from _util import codes_close, cuda, pmap, to_np

pytestmark = pytest.mark.gpu

TAU_ABS = 0.032
_POS = np.unique(F.decode_e4m3(np.arange(0x7F, dtype=np.uint8)))       # finite e4m3 magnitudes, sorted


def _valid_code_range(q):
    """The codes a drifted evaluation of the quotient q = a/s may give: those of every
    value within TAU_ABS code units of the oracle's fp32 quotient, i.e. the codes
    from enc(q - TAU_ABS) to enc(q + TAU_ABS) in value order (as decoded values)."""
    return F.decode_e4m3(F.encode_e4m3(q - TAU_ABS)), F.decode_e4m3(F.encode_e4m3(q + TAU_ABS))


def _oracle_expert(e, ids, xb):
    cfg = synth.MOE_PREFILL
    K, Ngu, Ndn, Kdn = cfg["K"], cfg["N_gu"], cfg["N_dn"], cfg["K_dn"]
    toks = np.nonzero(ids == e)[0]                   # pairs of expert e in increasing t·k + j
    bq1, sb1 = oracle.quantize_e4m3_blocks(synth.moe_prefill_expert_weight(1003, "gu", e, Ngu, K), 128, 128)
    bq2, sb2 = oracle.quantize_e4m3_blocks(synth.moe_prefill_expert_weight(1003, "dn", e, Ndn, Kdn), 128, 128)
    n = toks.size
    aq, sa = oracle.quantize_e4m3_blocks(xb[toks], 1, 128)
    seg = np.array([0, n])
    h = oracle.grouped_gemm_contiguous(aq, sa, bq1[None], sb1[None], seg)      # fp64
    q2, s2 = oracle.silu_mul_quantize(h)
    a32 = oracle.silu_mul(h).astype(np.float32)
    quot = (a32 / np.repeat(s2, 128, axis=1)).astype(np.float32).astype(np.float64)   # the quantizer's fl32(a/s)
    y = oracle.grouped_gemm_contiguous(q2, s2, bq2[None], sb2[None], seg)
    return dict(bq1=bq1, sb1=sb1, bq2=bq2, sb2=sb2, aq=aq, sa=sa, q2=q2, s2=s2, quot=quot, y=y)


def _allowance(q_gpu, s_gpu, o):
    """Σ_k |dq_gpu·s_gpu - dq_ref·s_ref|[r,k] · |B_deq[n,k]| for one expert's rows."""
    Ndn, Kdn = o["bq2"].shape
    d_in = np.abs(F.decode_e4m3(q_gpu) * np.repeat(s_gpu.astype(np.float64), 128, axis=1)
                  - F.decode_e4m3(o["q2"]) * np.repeat(o["s2"].astype(np.float64), 128, axis=1))
    out = np.zeros((q_gpu.shape[0], Ndn))
    rows = np.flatnonzero(d_in.any(axis=1))
    for kb in range(Kdn // 128):
        ks = slice(kb * 128, (kb + 1) * 128)
        if not d_in[rows, ks].any():
            continue
        bd = np.abs(F.decode_e4m3(o["bq2"][:, ks])) * o["sb2"][np.arange(Ndn) // 128, kb][:, None]
        out[rows] += d_in[rows, ks] @ bd.T
    return out


@pytest.mark.timeout(900)
def test_bench_prefill_step_every_output():
    cfg = synth.MOE_PREFILL
    T, E, k, Ndn = cfg["T"], cfg["E"], cfg["k"], cfg["N_dn"]

    def weight_fn(which, e, n, kk):
        return cuda(synth.moe_prefill_expert_weight(1003, which, e, n, kk))

    st = bench.setup_prefill(fgg, synth, torch, weight_fn=weight_fn)
    st["bufs"]["y"].fill_(float("nan"))
    bench.prefill_step(fgg, st)
    torch.cuda.synchronize()
    p, b = st["perm"], st["bufs"]
    offsets, counts = to_np(p["offsets"]).astype(np.int64), to_np(p["counts"])
    got = dict(s2r=to_np(p["src_to_row"]), r2s=to_np(p["row_to_src"]), a=to_np(p["a"]), sa=to_np(p["sa"]),
               a2=to_np(b["a2"]), s2=to_np(b["s2"]), y=to_np(b["y"]), out=to_np(b["out"]),
               gu_q=to_np(st["gu_q"]), gu_s=to_np(st["gu_s"]), dn_q=to_np(st["dn_q"]), dn_s=to_np(st["dn_s"]))
    del st, p, b
    torch.cuda.empty_cache()

    r = synth.moe_prefill_routing()
    ids, tw = r["topk_ids"], r["topk_w"]
    xb = synth.to_bf16_values(synth.moe_prefill_x())        # the bench's layer input is bf16
    ref = oracle.moe_permute(ids, E, 128)
    assert np.array_equal(offsets, ref["offsets"]) and np.array_equal(counts, ref["counts"])
    assert np.array_equal(got["s2r"], ref["src_to_row"])
    m_total = int(ref["offsets"][-1])
    assert np.array_equal(got["r2s"][:m_total], ref["row_to_src"][:m_total])

    def expert(e):
        o = _oracle_expert(e, ids, xb)
        rows = offsets[e] + np.arange(counts[e])
        o["allow"] = _allowance(got["a2"][rows], got["s2"][:, rows].T, o)
        return o

    res = pmap(expert, range(E))
    y_ref = np.zeros((m_total, Ndn))
    y_bound = np.zeros((m_total, Ndn))
    rows_all = []
    for e, o in enumerate(res):
        rows = offsets[e] + np.arange(counts[e])
        rows_all.append(rows)
        assert np.array_equal(got["gu_q"][e], o["bq1"]) and np.array_equal(got["gu_s"][e], o["sb1"]), e
        assert np.array_equal(got["dn_q"][e], o["bq2"]) and np.array_equal(got["dn_s"][e], o["sb2"]), e
        assert np.array_equal(got["a"][rows], o["aq"]) and np.array_equal(got["sa"][:, rows].T, o["sa"]), e
        # padding rows of the permuted activations: zero codes and scales
        pad = np.arange(offsets[e] + counts[e], offsets[e + 1])
        assert np.all(got["a"][pad] == 0) and np.all(got["sa"][:, pad] == 0)
        # requantized SiLU(gate)·up
        q, s = got["a2"][rows], got["s2"][:, rows].T
        np.testing.assert_allclose(s, o["s2"], rtol=2e-4, atol=0, err_msg=f"expert {e} requant scales")
        mism = q != o["q2"]
        lo, hi = _valid_code_range(o["quot"][mism])
        v = F.decode_e4m3(q[mism])
        bad = (v < lo) | (v > hi)
        assert not bad.any(), (
            f"expert {e}: {int(bad.sum())} of {q.size} codes outside the drift band "
            f"(of {int(mism.sum())} differing); oracle quotients {np.round(o['quot'][mism][bad][:8], 4).tolist()}, "
            f"gpu values {v[bad][:8].tolist()}")
        y_ref[rows] = o["y"]
        y_bound[rows] = o["allow"]
    del res
    rows_all = np.concatenate(rows_all)
    # down output (rows of the routed pairs; padding rows are not written)
    y_r = oracle.round_bf16(y_ref[rows_all])
    rms = float(np.sqrt(np.mean(y_r ** 2)))
    y = got["y"][rows_all]
    assert np.all(np.isfinite(y))
    excess = np.abs(y - y_r) - (1e-2 * (np.abs(y_r) + rms) + y_bound[rows_all] * (1 + 2.0 ** -7))
    assert not np.any(excess > 0), f"down output: {int((excess > 0).sum())} outputs outside the bound"
    pad_rows = np.setdiff1d(np.arange(m_total), rows_all)
    assert np.all(np.isnan(got["y"][pad_rows]))
    # combined layer output
    out_ref = oracle.round_bf16(oracle.moe_combine(oracle.round_bf16(y_ref), ref["src_to_row"], tw, T, k))
    slack = oracle.moe_combine(2.0 ** -8 * np.abs(oracle.round_bf16(y_ref)) + y_bound, ref["src_to_row"], tw, T, k)
    rms_o = float(np.sqrt(np.mean(out_ref ** 2)))
    excess = np.abs(got["out"] - out_ref) - (1e-2 * (np.abs(out_ref) + rms_o) + slack)
    assert not np.any(excess > 0), f"combined output: {int((excess > 0).sum())} outputs outside the bound"
    # and the bound is not what carries the comparison: almost every output meets the plain tolerance
    plain = np.abs(got["out"] - out_ref) <= 1e-2 * (np.abs(out_ref) + rms_o)
    assert plain.mean() > 0.999, plain.mean()
