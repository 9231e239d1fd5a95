"""GPU parity for the grouped / dense / masked / W4A4 GEMMs against the oracle.

Tolerance (floating point): |y - y_ref| <= 1e-2 · (|y_ref| + rms(y_ref)), with
y_ref the oracle's fp64 result rounded to bf16.  Padding rows must be exactly
zero; one group must equal the dense call bit for bit; runs are deterministic.
Every test compares every output it checks: the small cases, the persistent
multi-tile cases (test_gpu_persistent.py) and the full-size dense, decode and
W4A4 shapes (the oracle runs expert by expert or row block by row block on a
thread pool); the full prefill chain is in test_gpu_prefill_chain.py."""

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import oracle
import synth
from oracle import formats as F
from _util import codes_close, cuda, pmap, to_np, tol_check

pytestmark = pytest.mark.gpu


def _quant_weights_gpu(w_np, qdesc):
    """Quantize a [G, N, K] weight stack on the GPU, expert by expert."""
    G, N, K = w_np.shape
    outs, scales = [], []
    for e in range(G):
        q, s = fgg.quantize_blockwise(cuda(w_np[e]), qdesc)
        outs.append(q)
        scales.append(s)
    return torch.stack(outs), torch.stack(scales)


def _quant_weights_oracle(w_np):
    G, N, K = w_np.shape
    bq = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, N // 128, K // 128), np.float32)
    for e in range(G):
        bq[e], sb[e] = oracle.quantize_e4m3_blocks(w_np[e], 128, 128)
    return bq, sb


# ------------------------------------------------------------ one-hot probes

def test_one_hot_probe_contiguous():
    """A single 1.0 at (r, k) in A and at (n, k) of expert g in B lands on
    exactly (r, n), scaled by the distinct power-of-two block scales that
    belong to (r, k/128) and (g, n/128, k/128)."""
    G, N, K = 3, 256, 512
    offsets = np.array([0, 128, 128, 384], np.int32)      # expert 1 is empty
    M = 384
    for (r, n, k, g) in [(0, 0, 0, 0), (127, 255, 511, 0), (130, 17, 300, 2), (383, 128, 129, 2), (200, 64, 64, 2),
                         (5, 3, 3, 2), (300, 40, 500, 0)]:
        a = np.zeros((M, K), np.uint8)
        a[r, k] = 0x38
        b = np.zeros((G, N, K), np.uint8)
        b[g, n, k] = 0x38
        sa = np.ldexp(1.0, (np.arange(M)[None, :] % 7) + 3 * np.arange(K // 128)[:, None] - 8).astype(np.float32)
        sb = np.ldexp(1.0, np.arange(G * (N // 128) * (K // 128)).reshape(G, N // 128, K // 128) % 11 - 5).astype(np.float32)
        y = to_np(fgg.grouped_gemm_scaled(cuda(a), cuda(sa), cuda(b), cuda(sb), offsets=cuda(offsets)))
        expect = np.zeros((M, N))
        if np.searchsorted(offsets, r, side="right") - 1 == g:    # row r belongs to expert g
            expect[r, n] = sa[k // 128, r] * sb[g, n // 128, k // 128]
        assert np.array_equal(y, expect), (r, n, k, g)


def test_one_hot_probe_masked_fp4():
    """E2M1 operand layout, nibble order and per-32 E8M0 scale placement."""
    G, M, N, K = 2, 16, 128, 256
    masked = np.array([16, 9], np.int32)
    for (g, m, n, k) in [(0, 0, 0, 0), (0, 15, 127, 255), (1, 8, 33, 31), (1, 3, 64, 32), (0, 5, 16, 161), (1, 0, 1, 95)]:
        a = np.zeros((G, M, K), np.uint8)
        a[g, m, k] = 0x38
        b = np.zeros((G, N, K // 2), np.uint8)
        b[g, n, k // 2] = 0x2 << (4 * (k % 2))             # 1.0 in the nibble of element k
        sa = np.ldexp(1.0, np.arange(G * (K // 128) * M).reshape(G, K // 128, M) % 5 - 2).astype(np.float32)
        be = (127 + (np.arange(G * N * (K // 32)).reshape(G, N, K // 32) % 9) - 4).astype(np.uint8)
        y = to_np(fgg.grouped_gemm_scaled(cuda(a), cuda(sa), cuda(b), cuda(be), masked_m=cuda(masked),
                                          b_qdesc=fgg.Q_E2M1_E8M0_1x32))
        expect = np.zeros((G, M, N))
        expect[g, m, n] = sa[g, k // 128, m] * 2.0 ** (int(be[g, n, k // 32]) - 127)
        for gg in range(G):
            mm = masked[gg]
            assert np.array_equal(y[gg, :mm], expect[gg, :mm]), (g, m, n, k)


# ------------------------------------------------------- contiguous / dense

def _contig_case(seed, counts, N, K):
    G = len(counts)
    padded = [-(-c // 128) * 128 for c in counts]
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    M = int(offsets[-1]) + 64                 # extra rows beyond offsets[G] are never touched
    g = synth.rng(seed)
    x = synth.normal(g, (M, K))
    for e in range(G):                         # padding rows hold zeros, as after the permute
        x[offsets[e] + counts[e]:offsets[e + 1]] = 0
    w = synth.normal(g, (G, N, K), 0.02)
    return x, w, offsets


@pytest.mark.parametrize("counts,N,K", [([5, 0, 300, 128], 256, 512), ([1], 128, 128), ([129, 1000], 384, 1024)])
def test_grouped_contiguous_small(counts, N, K):
    x, w, offsets = _contig_case(len(counts) * 31 + N, counts, N, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    d = torch.full((x.shape[0], N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets), out=d)
    y = to_np(d)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = _quant_weights_oracle(w)
    assert np.array_equal(to_np(xq), aq_r) and np.array_equal(to_np(bq), bq_r)
    mt = int(offsets[-1])
    ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(aq_r, sa_r, bq_r, sb_r, offsets))[:mt]
    tol_check(y[:mt], ref, what="grouped contiguous")
    for e in range(len(counts)):                               # padding rows are exactly +0
        pad = y[offsets[e] + counts[e]:offsets[e + 1]]
        assert np.all(pad == 0) and not np.any(np.signbit(pad))
    assert np.all(np.isnan(y[mt:]))                            # rows >= offsets[G] untouched


_FRAG_COUNTS = [1, 15, 16, 17, 32, 33, 48, 63, 64, 65, 80, 81, 96, 112, 113, 127, 128, 129]


def _valid_rows(offsets, masked):
    """Rows [offsets[e], offsets[e] + clamp(masked[e], 0, segment length)) per group."""
    rows = []
    for e in range(len(masked)):
        n = min(max(int(masked[e]), 0), int(offsets[e + 1] - offsets[e]))
        rows.extend(range(int(offsets[e]), int(offsets[e]) + n))
    return np.array(rows, np.int64)


@pytest.mark.parametrize("counts,masked,N,K", [
    ([5, 0, 300, 128], [5, 0, 300, 128], 256, 512),        # tiles with 5 and 44 real rows
    ([5, 0, 300, 128], [2000, 7, -3, 64], 256, 512),       # clamped above / below, half tile
    ([129, 1000], [129, 1000], 384, 1024),
    ([64, 65], [64, 65], 128, 256),                        # exactly one busy row half, and one more row
    # every 16-row fragment boundary of both row halves of a tile (a wave computes only
    # the fragments that hold real rows)
    (_FRAG_COUNTS, _FRAG_COUNTS, 256, 384)])
def test_grouped_contiguous_valid_counts(counts, masked, N, K):
    """Per-group real row counts (masked_m with the contiguous layout): the rows
    they cover equal the unmasked call bit for bit; padding rows past them are
    not written."""
    x, w, offsets = _contig_case(len(counts) * 37 + N, counts, N, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    full = to_np(fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets)))
    d = torch.full((x.shape[0], N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets), masked_m=cuda(np.array(masked, np.int32)),
                            out=d)
    y = to_np(d)
    rows = _valid_rows(offsets, masked)
    assert np.array_equal(y[rows], full[rows])
    rest = np.setdiff1d(np.arange(x.shape[0]), rows)
    assert np.all(np.isnan(y[rest]))


def test_k_zero_gives_zeros():
    """K == 0: empty sums, so every computed output is +0 (and the SiLU requant of a
    zero row is codes 0 with scale 1); nothing is fetched."""
    G, N, M = 2, 256, 300
    offsets = np.array([0, 128, 256], np.int32)
    a = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((0, M), dtype=torch.float32, device="cuda")
    b = torch.zeros((G, N, 0), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((G, N // 128, 0), dtype=torch.float32, device="cuda")
    d = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(a, sa, b, sb, offsets=cuda(offsets), out=d)
    y = to_np(d)
    assert np.all(y[:256] == 0) and not np.any(np.signbit(y[:256])) and np.all(np.isnan(y[256:]))
    yd = to_np(fgg.scaled_gemm(a, sa, b[0], sb[0]))
    assert yd.shape == (M, N) and np.all(yd == 0)
    q = torch.full((M, N // 2), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((N // 256, M), -3.0, dtype=torch.float32, device="cuda")
    fgg.grouped_gemm_silu_quantize(a, sa, b, sb, cuda(offsets), out=q, scales=s)
    q, s = to_np(q), to_np(s)
    assert np.all(q[:256] == 0) and np.all(s[:, :256] == 1.0)
    assert np.all(q[256:] == 0xAB) and np.all(s[:, 256:] == -3.0)


def test_grouped_contiguous_max_groups():
    """1024 experts (the limit), almost all empty, the used ones spread over the
    whole id range: every tile finds its expert in the workgroup's group table."""
    G, N, K = 1024, 128, 128
    counts = [0] * G
    for e, c in ((0, 3), (1, 130), (511, 1), (512, 128), (1000, 200), (1023, 77)):
        counts[e] = c
    x, w, offsets = _contig_case(4242, counts, N, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    y = to_np(fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets)))
    yc = to_np(fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets),
                                       masked_m=cuda(np.array(counts, np.int32))))
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    mt = int(offsets[-1])
    used = [e for e in range(G) if counts[e] > 0]
    for e in used:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        bq_r, sb_r = oracle.quantize_e4m3_blocks(w[e], 128, 128)
        ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(aq_r[lo:hi], sa_r[lo:hi], bq_r[None], sb_r[None],
                                                               np.array([0, hi - lo])))
        tol_check(y[lo:hi], ref, what=f"expert {e} of 1024")
        assert np.array_equal(yc[lo:lo + counts[e]], y[lo:lo + counts[e]])
    assert mt == sum(-(-c // 128) * 128 for c in counts)


def test_grouped_contiguous_max_k():
    """K = 16384 (the contiguous layout's limit: 128 K blocks)."""
    counts, N, K = [130, 5], 256, 16384
    x, w, offsets = _contig_case(99, counts, N, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    y = to_np(fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(offsets)))
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = _quant_weights_oracle(w)
    mt = int(offsets[-1])
    ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(aq_r, sa_r, bq_r, sb_r, offsets))[:mt]
    tol_check(y[:mt], ref, what="grouped contiguous K=16384")


@pytest.mark.parametrize("M,N,K", [(500, 256, 1024), (128, 128, 128), (1, 128, 256)])
def test_dense_small_and_one_group_identity(M, N, K):
    g = synth.rng(M + N + K)
    x = synth.normal(g, (M, K))
    w = synth.normal(g, (N, K), 0.02)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = fgg.quantize_blockwise(cuda(w), fgg.Q_E4M3_128x128)
    y = fgg.scaled_gemm(xq, xs, bq, sb)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = oracle.quantize_e4m3_blocks(w, 128, 128)
    ref = oracle.round_bf16(oracle.scaled_gemm_dense(aq_r, sa_r, bq_r, sb_r))
    tol_check(to_np(y), ref, what="dense")
    # the grouped call with one group covering [0, M) is the same computation
    y1 = fgg.grouped_gemm_scaled(xq, xs, bq[None], sb[None], offsets=cuda(np.array([0, M], np.int32)))
    if M % 128 == 0:
        assert torch.equal(y1, y)
    else:
        assert torch.equal(y1[:M], y[:M])


def test_dense_full_size_every_output_and_deterministic():
    w = synth.dense()
    M, N, K = w["M"], w["N"], w["K"]
    xq, xs = fgg.quantize_blockwise(cuda(w["x"]), fgg.Q_E4M3_1x128)
    bq, sb = fgg.quantize_blockwise(cuda(w["w"]), fgg.Q_E4M3_128x128)
    y = fgg.scaled_gemm(xq, xs, bq, sb)
    y2 = fgg.scaled_gemm(xq, xs, bq, sb)
    assert torch.equal(y, y2)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(w["x"], 1, 128)
    bq_r, sb_r = oracle.quantize_e4m3_blocks(w["w"], 128, 128)
    assert np.array_equal(to_np(xq), aq_r) and np.array_equal(to_np(bq), bq_r)
    ref = oracle.round_bf16(oracle.scaled_gemm_dense(aq_r, sa_r, bq_r, sb_r))
    tol_check(to_np(y), ref, what="dense 4096x4096x7168, every output")


# ------------------------------------------------------------- MoE chains

def _moe_chain_gpu(x, topk_ids, topk_w, E, wq_gu, ws_gu, wq_dn=None, ws_dn=None, use_counts=False):
    """use_counts: both GEMMs get the permute's counts, so padding rows are skipped
    (and their outputs left unwritten)."""
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    perm = fgg.moe_permute(cuda(topk_ids), E, 128, xq=xq, xs=xs)
    mm = perm["counts"] if use_counts else None
    h = fgg.grouped_gemm_scaled(perm["a"], perm["sa"], wq_gu, ws_gu, offsets=perm["offsets"], masked_m=mm)
    if wq_dn is None:
        y = h
    else:
        a2, s2 = fgg.quantize_blockwise(h, fgg.Q_E4M3_1x128, silu_mul=True)
        y = fgg.grouped_gemm_scaled(a2, s2, wq_dn, ws_dn, offsets=perm["offsets"], masked_m=mm)
    out = fgg.moe_combine(y, perm["src_to_row"], cuda(topk_w))
    return out, perm, h, y


def test_tiny_moe_end_to_end():
    w = synth.tiny_moe()
    T, E, k = w["T"], w["E"], w["k"]
    bq, sb = _quant_weights_gpu(w["w"], fgg.Q_E4M3_128x128)
    out, perm, h, _ = _moe_chain_gpu(w["x"], w["topk_ids"], w["topk_w"], E, bq, sb)
    # oracle chain
    aq_r, sa_r = oracle.quantize_e4m3_blocks(w["x"], 1, 128)
    p = oracle.moe_permute(w["topk_ids"], E, 128)
    mt = int(p["offsets"][-1])
    a_r, s_r = oracle.gather_permuted(p["row_to_src"], mt, k, aq_r, sa_r)
    bq_r, sb_r = _quant_weights_oracle(w["w"])
    h_r = oracle.round_bf16(oracle.grouped_gemm_contiguous(a_r, s_r, bq_r, sb_r, p["offsets"]))
    tol_check(to_np(h)[:mt], h_r, what="tiny MoE expert outputs")
    out_r = oracle.round_bf16(oracle.moe_combine(h_r, p["src_to_row"], w["topk_w"], T, k))
    tol_check(to_np(out), out_r, what="tiny MoE combined output")
    assert out.shape == (64, 512)


def test_moe_prefill_full_size_sampled():
    cfg = synth.MOE_PREFILL
    T, K, E, k = cfg["T"], cfg["K"], cfg["E"], cfg["k"]
    Ngu, Ndn, Kdn = cfg["N_gu"], cfg["N_dn"], cfg["K_dn"]
    r = synth.moe_prefill_routing()
    x = synth.moe_prefill_x()
    gu_q, gu_s, dn_q, dn_s = [], [], [], []
    w_keep = {}
    sample_experts = [0, 7, 31]
    for e in range(E):
        wgu = synth.moe_prefill_expert_weight(1003, "gu", e, Ngu, K)
        wdn = synth.moe_prefill_expert_weight(1003, "dn", e, Ndn, Kdn)
        q, s = fgg.quantize_blockwise(cuda(wgu), fgg.Q_E4M3_128x128)
        gu_q.append(q); gu_s.append(s)
        q, s = fgg.quantize_blockwise(cuda(wdn), fgg.Q_E4M3_128x128)
        dn_q.append(q); dn_s.append(s)
        if e in sample_experts:
            w_keep[e] = (wgu, wdn)
    gu_q, gu_s = torch.stack(gu_q), torch.stack(gu_s)
    dn_q, dn_s = torch.stack(dn_q), torch.stack(dn_s)
    out, perm, h, y = _moe_chain_gpu(x, r["topk_ids"], r["topk_w"], E, gu_q, gu_s, dn_q, dn_s)
    offsets = to_np(perm["offsets"]).astype(np.int64)
    counts = to_np(perm["counts"])
    r2s = to_np(perm["row_to_src"])
    a_all = to_np(perm["a"])
    sa_all = to_np(perm["sa"])
    h_np = to_np(h)
    for e in sample_experts:
        rows = offsets[e] + np.unique(np.linspace(0, counts[e] - 1, 6).astype(np.int64))
        rows = np.concatenate([rows, [offsets[e + 1] - 1]])                 # a padding row
        wgu, wdn = w_keep[e]
        bq_r, sb_r = oracle.quantize_e4m3_blocks(wgu, 128, 128)
        assert np.array_equal(to_np(gu_q[e]), bq_r)
        a_r = a_all[rows]
        sa_r = sa_all[:, rows].T
        # the permuted rows are the token rows quantized by the oracle
        toks = r2s[rows] // k
        valid = r2s[rows] >= 0
        aq_tok, sa_tok = oracle.quantize_e4m3_blocks(x[toks[valid]], 1, 128)
        assert np.array_equal(a_r[valid], aq_tok) and np.array_equal(sa_r[valid], sa_tok)
        h_ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(
            a_r, sa_r, bq_r[None], sb_r[None], np.array([0, len(rows)])))
        tol_check(h_np[rows], h_ref, what=f"prefill gate-up expert {e}")
        assert np.all(h_np[offsets[e + 1] - 1] == 0) or counts[e] % 128 == 0
        # down projection of the same rows from the GPU's own gate-up output
        a2_r, s2_r = oracle.silu_mul_quantize(h_np[rows].astype(np.float64))
        bq2, sb2 = oracle.quantize_e4m3_blocks(wdn, 128, 128)
        y_ref = oracle.round_bf16(oracle.grouped_gemm_contiguous(
            a2_r, s2_r, bq2[None], sb2[None], np.array([0, len(rows)])))
        tol_check(to_np(y)[rows], y_ref, what=f"prefill down expert {e}")
    # the same chain with the permute's counts given to both GEMMs: padding rows are
    # skipped, and the combined output is identical bit for bit
    out_c, _, _, _ = _moe_chain_gpu(x, r["topk_ids"], r["topk_w"], E, gu_q, gu_s, dn_q, dn_s, use_counts=True)
    assert torch.equal(out_c, out)
    del out_c
    # combine for a sample of tokens, from the GPU's own expert outputs
    toks = np.arange(0, T, 997)
    y_np = to_np(y)
    s2r = to_np(perm["src_to_row"])
    ref = oracle.round_bf16(oracle.moe_combine(y_np, s2r.reshape(T, k)[toks].reshape(-1),
                                               r["topk_w"][toks], len(toks), k))
    tol_check(to_np(out)[toks], ref, what="prefill combine")


# ----------------------------------------------------------------- masked

def _masked_case(G, M, N, K, seed, masked=None):
    g = synth.rng(seed)
    if masked is None:
        masked = g.integers(1, M + 1, size=G).astype(np.int32)
    x = synth.normal(g, (G, M, K))
    w = synth.normal(g, (G, N, K), 0.02)
    return x, w, masked


def _quant_masked_a_gpu(x):
    G, M, K = x.shape
    aq, sa = fgg.quantize_blockwise(cuda(x.reshape(G * M, K)), fgg.Q_E4M3_1x128)
    # [K/128, G*M] -> [G, K/128, M]
    sa = sa.reshape(K // 128, G, M).permute(1, 0, 2).contiguous()
    return aq.reshape(G, M, K), sa


@pytest.mark.parametrize("G,M,N,K,masked", [(4, 16, 256, 512, [16, 1, 0, 7]), (3, 5, 128, 128, [5, 5, 2]),
                                            (2, 16, 640, 1024, None)])
def test_masked_fp4_small(G, M, N, K, masked):
    x, w, mm = _masked_case(G, M, N, K, G * 100 + N, None if masked is None else np.array(masked, np.int32))
    aq, sa = _quant_masked_a_gpu(x)
    bq, be = _quant_weights_gpu(w, fgg.Q_E2M1_E8M0_1x32)
    d = torch.full((G, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(aq, sa, bq, be, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32, out=d)
    y = to_np(d)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x.reshape(G * M, K), 1, 128)
    aq_r, sa_r = aq_r.reshape(G, M, K), sa_r.reshape(G, M, K // 128)
    bc = np.empty((G, N, K), np.uint8)
    be_r = np.empty((G, N, K // 32), np.uint8)
    for e in range(G):
        bc[e], be_r[e] = oracle.quantize_e2m1_e8m0_groups(w[e], 32)
    bp_r = F.pack_e2m1x2(bc)
    assert np.array_equal(to_np(bq), bp_r) and np.array_equal(to_np(be), be_r)
    ref = oracle.round_bf16(oracle.grouped_gemm_masked(aq_r, sa_r, bp_r, be_r, mm))
    for e in range(G):
        m = int(mm[e])
        tol_check(y[e, :m], ref[e, :m], what=f"masked fp4 group {e}")
        assert np.all(np.isnan(y[e, m:]))                       # rows >= masked_m untouched


def test_masked_fp4_full_size_every_output():
    """Decode shape (32 experts x 1..16 rows, N 4096, K 7168): every expert's every
    real row against the oracle; rows >= masked_m are never written."""
    wl = synth.moe_decode(with_weights=False)
    G, M, N, K = wl["G"], wl["M_max"], wl["N"], wl["K"]
    mm = wl["masked_m"]
    aq, sa = _quant_masked_a_gpu(wl["x"])
    bq = torch.empty((G, N, K // 2), dtype=torch.uint8, device="cuda")
    be = torch.empty((G, N, K // 32), dtype=torch.uint8, device="cuda")
    for e in range(G):
        fgg.quantize_blockwise(cuda(synth.moe_decode_expert_weight(1004, e, N, K)), fgg.Q_E2M1_E8M0_1x32,
                               out=bq[e], scales=be[e])
    d = torch.full((G, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(aq, sa, bq, be, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32, out=d)
    y2 = fgg.grouped_gemm_scaled(aq, sa, bq, be, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32)
    for e in range(G):
        assert torch.equal(d[e, :int(mm[e])], y2[e, :int(mm[e])])
    y, bq_np, be_np = to_np(d), to_np(bq), to_np(be)

    def expert(e):
        m = int(mm[e])
        aq_r, sa_r = oracle.quantize_e4m3_blocks(wl["x"][e], 1, 128)
        bc, be_r = oracle.quantize_e2m1_e8m0_groups(synth.moe_decode_expert_weight(1004, e, N, K), 32)
        bp_r = F.pack_e2m1x2(bc)
        codes_ok = np.array_equal(bq_np[e], bp_r) and np.array_equal(be_np[e], be_r)
        ref = oracle.round_bf16(oracle.grouped_gemm_masked(aq_r[None], sa_r[None], bp_r[None], be_r[None],
                                                           np.array([m])))
        return codes_ok, ref[0, :m]

    res = pmap(expert, range(G))
    assert all(ok for ok, _ in res), "decode weight codes differ from the oracle's"
    tol_check(np.concatenate([y[e, :int(mm[e])] for e in range(G)]), np.concatenate([r for _, r in res]),
              what="decode 32 experts, every output")
    for e in range(G):
        assert np.all(np.isnan(y[e, int(mm[e]):]))


@pytest.mark.parametrize("G,M,N,K,masked", [(3, 16, 256, 1024, [16, 0, 9]), (2, 7, 128, 384, [7, 3]),
                                            (1, 16, 128, 640, [1])])
def test_masked_fp4_tiled_equals_plain(G, M, N, K, masked):
    """Weights re-laid out by pack_fp4_weights: the packer matches the oracle's
    statement of the layout byte for byte (including the 127 padding of partial
    scale spans), and the masked GEMM on the tiled weights equals the one on the
    plain weights bit for bit (the same operands reach the same MFMAs)."""
    x, w, _ = _masked_case(G, M, N, K, G * 77 + N + K)
    mm = np.array(masked, np.int32)
    aq, sa = _quant_masked_a_gpu(x)
    bq, be = _quant_weights_gpu(w, fgg.Q_E2M1_E8M0_1x32)
    bt, st = fgg.pack_fp4_weights(bq, be)
    codes_r, scales_r = oracle.tile_fp4_weights(to_np(bq), to_np(be))
    assert np.array_equal(to_np(bt).reshape(-1), codes_r) and np.array_equal(to_np(st).reshape(-1), scales_r)
    d1 = torch.full((G, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    d2 = torch.full((G, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fgg.grouped_gemm_scaled(aq, sa, bq, be, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32, out=d1)
    fgg.grouped_gemm_scaled(aq, sa, bt, st, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32_TILED, out=d2, n=N)
    y1, y2 = to_np(d1), to_np(d2)
    for e in range(G):
        m = int(mm[e])
        assert np.array_equal(y2[e, :m], y1[e, :m])
        assert np.all(np.isnan(y2[e, m:]))


def test_masked_fp4_tiled_full_size():
    """Decode shape (32 experts, N 4096, K 7168): tiled and plain layouts give the
    same outputs bit for bit; sampled tiles of the packed weights match the oracle."""
    wl = synth.moe_decode(with_weights=False)
    G, M, N, K = wl["G"], wl["M_max"], wl["N"], wl["K"]
    mm = wl["masked_m"]
    aq, sa = _quant_masked_a_gpu(wl["x"])
    bq = torch.empty((G, N, K // 2), dtype=torch.uint8, device="cuda")
    be = torch.empty((G, N, K // 32), dtype=torch.uint8, device="cuda")
    for e in range(G):
        we = synth.moe_decode_expert_weight(1004, e, N, K)
        fgg.quantize_blockwise(cuda(we), fgg.Q_E2M1_E8M0_1x32, out=bq[e], scales=be[e])
    bt, st = fgg.pack_fp4_weights(bq, be)
    y1 = fgg.grouped_gemm_scaled(aq, sa, bq, be, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32)
    y2 = fgg.grouped_gemm_scaled(aq, sa, bt, st, masked_m=cuda(mm), b_qdesc=fgg.Q_E2M1_E8M0_1x32_TILED, n=N)
    for e in range(G):
        assert torch.equal(y2[e, :int(mm[e])], y1[e, :int(mm[e])])
    # experts 5 and 30, rows 1024..1055 (two 16-row groups), all K, against the oracle's layout
    for e in (5, 30):
        cr, sr = oracle.tile_fp4_weights(to_np(bq[e:e + 1, 1024:1056]), to_np(be[e:e + 1, 1024:1056]))
        tile_bytes, span_bytes = (K // 128) * 1024, ((K // 32 + 15) // 16) * 256
        g0 = e * (N // 16) + 1024 // 16                      # first 16-row group of the sample
        got_c = to_np(bt).reshape(-1)[g0 * tile_bytes:(g0 + 2) * tile_bytes]
        got_s = to_np(st).reshape(-1)[g0 * span_bytes:(g0 + 2) * span_bytes]
        assert np.array_equal(got_c, cr) and np.array_equal(got_s, sr)


def test_masked_fp8_equals_contiguous():
    G, M, N, K = 3, 16, 256, 512
    x, w, mm = _masked_case(G, M, N, K, 4242, np.array([16, 3, 11], np.int32))
    aq, sa = _quant_masked_a_gpu(x)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    y_m = to_np(fgg.grouped_gemm_scaled(aq, sa, bq, sb, masked_m=cuda(mm), b_qdesc=fgg.Q_E4M3_128x128))
    # the same rows laid out contiguously, one 128-row segment per group
    xc = np.zeros((G * 128, K), np.float32)
    for e in range(G):
        xc[e * 128:e * 128 + M] = x[e]
    xq, xs = fgg.quantize_blockwise(cuda(xc), fgg.Q_E4M3_1x128)
    y_c = to_np(fgg.grouped_gemm_scaled(xq, xs, bq, sb, offsets=cuda(np.arange(G + 1, dtype=np.int32) * 128)))
    for e in range(G):
        m = int(mm[e])
        assert np.array_equal(y_m[e, :m], y_c[e * 128:e * 128 + m])


# ------------------------------------------------------------------- W4A4

def _w4a4_run(wl, rows=None):
    M, N, K = wl["M"], wl["N"], wl["K"]
    xq, xs = fgg.quantize_blockwise(cuda(wl["x"]), fgg.Q_E2M1_1x16)
    wq, ws = fgg.quantize_blockwise(cuda(wl["w"]), fgg.Q_E2M1_1x16)
    y = fgg.scaled_gemm(xq, xs, wq, ws, qdesc="w4a4", x_bf16=cuda(wl["x"], torch.bfloat16),
                        l_down=cuda(wl["l_down"], torch.bfloat16), l_up=cuda(wl["l_up"], torch.bfloat16),
                        bias=cuda(wl["bias"], torch.bfloat16))
    rows = np.arange(M) if rows is None else rows
    qx_r, sx_r = oracle.quantize_e2m1_fp32_groups(wl["x"][rows], 16)
    qw_r, sw_r = oracle.quantize_e2m1_fp32_groups(wl["w"], 16)
    assert np.array_equal(to_np(xq)[rows], F.pack_e2m1x2(qx_r)) and np.array_equal(to_np(wq), F.pack_e2m1x2(qw_r))
    # the oracle in 256-row blocks side by side
    blocks = [slice(r, r + 256) for r in range(0, len(rows), 256)]
    ref = np.concatenate(pmap(lambda b: oracle.w4a4_lowrank_gemm(
        qx_r[b], sx_r[b], qw_r, sw_r, wl["x"][rows][b], wl["l_down"], wl["l_up"], wl["bias"]), blocks))
    return to_np(y)[rows], oracle.round_bf16(ref)


def test_w4a4_small():
    wl = synth.w4a4(seed=77, M=256, N=384, K=512)
    y, ref = _w4a4_run(wl)
    tol_check(y, ref, what="w4a4 small")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(384, 640, 256), (640, 384, 128), (1152, 896, 256)])
def test_w4a4_partial_tiles(M, N, K):
    # 256 x 192 workgroup tiles: partial tiles in M and N, fewer than four tile rows in the
    # last raster group, tile counts that are not a multiple of the XCD count
    wl = synth.w4a4(seed=79 + M, M=M, N=N, K=K)
    y, ref = _w4a4_run(wl)
    tol_check(y, ref, what=f"w4a4 {M}x{N}x{K}")


def test_w4a4_no_epilogue():
    """No low-rank branch and no bias: the plain W4A4 product."""
    wl = synth.w4a4(seed=78, M=128, N=256, K=384)
    M, N, K = 128, 256, 384
    xq, xs = fgg.quantize_blockwise(cuda(wl["x"]), fgg.Q_E2M1_1x16)
    wq, ws = fgg.quantize_blockwise(cuda(wl["w"]), fgg.Q_E2M1_1x16)
    y = to_np(fgg.scaled_gemm(xq, xs, wq, ws, qdesc="w4a4"))
    qx_r, sx_r = oracle.quantize_e2m1_fp32_groups(wl["x"], 16)
    qw_r, sw_r = oracle.quantize_e2m1_fp32_groups(wl["w"], 16)
    assert np.array_equal(to_np(xq), F.pack_e2m1x2(qx_r)) and np.array_equal(to_np(wq), F.pack_e2m1x2(qw_r))
    ref = oracle.round_bf16(oracle.w4a4_lowrank_gemm(qx_r, sx_r, qw_r, sw_r))
    tol_check(y, ref, what="w4a4 without epilogue")


def test_w4a4_full_size_every_output():
    wl = synth.w4a4()
    y, ref = _w4a4_run(wl)
    tol_check(y, ref, what="w4a4 4096x3072x3072, every output")


@pytest.mark.parametrize("M,N,K", [(128, 256, 384), (256, 128, 3072)])
def test_w4a4_lowrank_branch_alone(M, N, K):
    # all-zero FP4 codes: the block-scaled product vanishes and the output is the
    # low-rank term plus bias alone, so a mistake there cannot hide under the
    # tolerance of the (much larger) main product; K = 384 gives each of the four
    # K-split waves a range that is not a multiple of 128
    wl = synth.w4a4(seed=91, M=M, N=N, K=K)
    ld = wl["l_down"] * np.float32(20.0)           # make the rank term O(1)
    zq = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    zs = torch.ones((M, K // 16), dtype=torch.float32, device="cuda")
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.ones((N, K // 16), dtype=torch.float32, device="cuda")
    y = fgg.scaled_gemm(zq, zs, wq, ws, qdesc="w4a4", x_bf16=cuda(wl["x"], torch.bfloat16),
                        l_down=cuda(synth.to_bf16_values(ld), torch.bfloat16),
                        l_up=cuda(wl["l_up"], torch.bfloat16), bias=cuda(wl["bias"], torch.bfloat16))
    ref = oracle.round_bf16(oracle.w4a4_lowrank_gemm(
        np.zeros((M, K), np.uint8), np.ones((M, K // 16), np.float32), np.zeros((N, K), np.uint8),
        np.ones((N, K // 16), np.float32), wl["x"], synth.to_bf16_values(ld), wl["l_up"], wl["bias"]))
    assert np.abs(ref).max() > 0.1                  # the branch is really exercised
    tol_check(to_np(y), ref, what="w4a4 low-rank branch")


# ------------------------------------------------- fused gate-up + SiLU requant

def _silu_requant_close(q, s, q_r, s_r, h_ref, what):
    """Fused gate-up + SiLU requant against the oracle on the exact fp64 GEMM.
    The GPU's fp32 GEMM result differs from the exact one within the library's
    GEMM tolerance (large relative errors only where terms cancel to a tiny
    value), so the codes are compared after dequantization: both sides' half-step
    quantization error (2^-4 relative, 2^-10 of the scale near zero) plus that
    tolerance carried through SiLU(gate)*up.  Scales (group maxima) agree to
    2e-4 relative and almost every code is identical."""
    codes_close(q, q_r, s, s_r, rtol=2e-4, min_equal=0.995, max_step=None, what=what)
    a_ref = oracle.silu_mul(h_ref)
    rms = float(np.sqrt(np.mean(a_ref ** 2)))
    s_full, s_r_full = np.repeat(s, 128, axis=1), np.repeat(s_r, 128, axis=1)
    deq = F.decode_e4m3(q) * s_full
    deq_r = F.decode_e4m3(q_r) * s_r_full
    bound = 2.0 ** -3 * np.abs(a_ref) + 2.0 ** -9 * s_r_full + 1e-2 * (np.abs(a_ref) + rms)
    bad = np.abs(deq - deq_r) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} dequantized values outside tolerance"


@pytest.mark.parametrize("counts,I,K", [([5, 0, 300, 128], 128, 512), ([1], 128, 128), ([129, 1000], 256, 1024)])
def test_grouped_silu_quantize_small(counts, I, K):
    x, w, offsets = _contig_case(len(counts) * 17 + I + K, counts, 2 * I, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    M = x.shape[0]
    q = torch.full((M, I), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((I // 128, M), -3.0, dtype=torch.float32, device="cuda")
    fgg.grouped_gemm_silu_quantize(xq, xs, bq, sb, cuda(offsets), out=q, scales=s)
    q, s = to_np(q), to_np(s)
    aq_r, sa_r = oracle.quantize_e4m3_blocks(x, 1, 128)
    bq_r, sb_r = _quant_weights_oracle(w)
    mt = int(offsets[-1])
    h = oracle.grouped_gemm_contiguous(aq_r, sa_r, bq_r, sb_r, offsets)[:mt]   # fp64, not rounded
    q_r, s_r = oracle.silu_mul_quantize(h)
    _silu_requant_close(q[:mt], s[:, :mt].T, q_r, s_r, h, "fused gate-up SiLU requant")
    assert np.all(q[mt:] == 0xAB) and np.all(s[:, mt:] == -3.0)       # rows >= offsets[G] untouched
    for e in range(len(counts)):                                      # padding rows: zero codes, scale 1
        lo, hi = offsets[e] + counts[e], offsets[e + 1]
        assert np.all(q[lo:hi] == 0) and np.all(s[:, lo:hi] == 1.0)


@pytest.mark.parametrize("counts,masked,I,K", [([5, 0, 300, 128], [5, 0, 300, 128], 128, 512),
                                               ([5, 0, 300, 128], [2000, 7, -3, 64], 256, 512),
                                               (_FRAG_COUNTS, _FRAG_COUNTS, 128, 384)])
def test_grouped_silu_quantize_valid_counts(counts, masked, I, K):
    """Per-group real row counts: the rows they cover equal the call without
    counts bit for bit; codes and scales of padding rows are not written."""
    x, w, offsets = _contig_case(len(counts) * 19 + I + K, counts, 2 * I, K)
    xq, xs = fgg.quantize_blockwise(cuda(x), fgg.Q_E4M3_1x128)
    bq, sb = _quant_weights_gpu(w, fgg.Q_E4M3_128x128)
    M = x.shape[0]
    q0, s0 = fgg.grouped_gemm_silu_quantize(xq, xs, bq, sb, cuda(offsets))
    q = torch.full((M, I), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((I // 128, M), -3.0, dtype=torch.float32, device="cuda")
    fgg.grouped_gemm_silu_quantize(xq, xs, bq, sb, cuda(offsets), counts=cuda(np.array(masked, np.int32)),
                                   out=q, scales=s)
    q, s, q0, s0 = to_np(q), to_np(s), to_np(q0), to_np(s0)
    rows = _valid_rows(offsets, masked)
    assert np.array_equal(q[rows], q0[rows]) and np.array_equal(s[:, rows], s0[:, rows])
    rest = np.setdiff1d(np.arange(M), rows)
    assert np.all(q[rest] == 0xAB) and np.all(s[:, rest] == -3.0)


def test_grouped_silu_quantize_prefill_matches_separate_path():
    """Full prefill gate-up shape: the fused kernel against the separate GEMM +
    SiLU requant (bf16 H in between), and sampled rows against the oracle."""
    cfg = synth.MOE_PREFILL
    T, K, E, k, Ngu = cfg["T"], cfg["K"], cfg["E"], cfg["k"], cfg["N_gu"]
    r = synth.moe_prefill_routing()
    x = synth.moe_prefill_x()
    perm = fgg.moe_permute(cuda(r["topk_ids"]), E, 128, x=cuda(x, torch.bfloat16))
    gu_q, gu_s = [], []
    keep = {}
    for e in range(E):
        wgu = synth.moe_prefill_expert_weight(1003, "gu", e, Ngu, K)
        qq, ss = fgg.quantize_blockwise(cuda(wgu), fgg.Q_E4M3_128x128)
        gu_q.append(qq); gu_s.append(ss)
        if e in (3, 30):
            keep[e] = wgu
    gu_q, gu_s = torch.stack(gu_q), torch.stack(gu_s)
    offs = perm["offsets"]
    q, s = fgg.grouped_gemm_silu_quantize(perm["a"], perm["sa"], gu_q, gu_s, offs)
    # with the permute's counts (padding rows skipped): identical on the real rows
    qc, sc = fgg.grouped_gemm_silu_quantize(perm["a"], perm["sa"], gu_q, gu_s, offs, counts=perm["counts"])
    real = _valid_rows(to_np(offs), to_np(perm["counts"]))
    assert np.array_equal(to_np(qc)[real], to_np(q)[real]) and np.array_equal(to_np(sc)[:, real], to_np(s)[:, real])
    del qc, sc
    h = fgg.grouped_gemm_scaled(perm["a"], perm["sa"], gu_q, gu_s, offsets=offs)
    q2, s2 = fgg.quantize_blockwise(h, fgg.Q_E4M3_1x128, silu_mul=True, rows_dev=offs[E:])
    mt = int(to_np(offs)[E])
    q, s, q2, s2 = to_np(q)[:mt], to_np(s)[:, :mt], to_np(q2)[:mt], to_np(s2)[:, :mt]
    # the separate path rounds gate and up to bf16 (each within 2^-9 relative) before
    # SiLU, whose relative sensitivity d ln SiLU(g) / d ln g = 1 + g (1 - sigmoid(g))
    # grows to |1 + g| for negative g: scales agree to ~1%, codes to one step, and a
    # few percent of the codes sit across a rounding boundary
    codes_close(q, q2, s.T, s2.T, rtol=2e-2, min_equal=0.9, max_step=1, what="fused vs separate path")
    offsets = to_np(offs).astype(np.int64)
    counts = to_np(perm["counts"])
    a_all, sa_all = to_np(perm["a"]), to_np(perm["sa"])
    for e, wgu in keep.items():
        rows = offsets[e] + np.unique(np.linspace(0, counts[e] - 1, 5).astype(np.int64))
        bq_r, sb_r = oracle.quantize_e4m3_blocks(wgu, 128, 128)
        h_r = oracle.grouped_gemm_contiguous(a_all[rows], sa_all[:, rows].T, bq_r[None], sb_r[None],
                                             np.array([0, len(rows)]))
        q_r, s_r = oracle.silu_mul_quantize(h_r)
        _silu_requant_close(q[rows], s[:, rows].T, q_r, s_r, h_r, f"fused gate-up expert {e}")
