#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 MoE layer hot path on one MI355X.

One step = one pass of the prefill MoE layer (T=8192 tokens, hidden 7168, 32
local experts of 256, top-8, Zipf(1.1)-ragged segments padded to 128):
  moe_permute with the 1x128 e4m3 quantization of X fused into its gather
  -> gate-up grouped GEMM (N=4096) with SiLU(gate)*up and the e4m3 1x128
  requantization fused into its epilogue -> down grouped GEMM (N=7168,
  K=2048) -> gate-weighted combine (bf16 [8192, 7168]).
Inputs are resident in HBM before timing starts; expert weights are quantized
once, untimed (offline weight quantization).

value = useful grouped-GEMM FLOPs of the step (2·8192·(4096·7168 + 7168·2048)
= 721.6 GFLOP) / measured step time, in TFLOP/s.  The roofline object covers
the dominant kernel (the gate-up grouped GEMM), timed with HIP events on the
stream it runs on, in a second pass of as many steps (the step time is taken
from steps without events between their kernels).  The decode workload (32 experts × 1-16 tokens, FP4
weights) and the dense / W4A4 shapes are measured in the same run and
reported under "secondary".

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "grouped-GEMM TFLOPS (% FP8/FP4 MFMA peak); decode GB/s (% HBM peak)"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense FP4 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def measured_traffic(root):
    """HBM bytes per launch of the gate-up GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE record, scaled by the copy calibration; None when
    the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(root, "profiles", "gemm_fp8_contig_gate_up_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for s in rec["sources"]:
        h.update(open(os.path.join(root, s), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return (rec["fetch_size_kib"] * rec["fetch_factor"] + rec["write_size_kib"] * rec["write_factor"]) * 1024.0


def _sync():
    import torch
    torch.cuda.synchronize()


def roofline_entry(kernel, flops, nbytes, seconds, mfma_peak_tflops, how):
    """Both roofline fractions of one launch: achieved algorithmic FLOP/s against the
    matrix-core peak of its dtype and algorithmic bytes/s against HBM.  The bound is
    the side with the larger minimum time (arithmetic intensity against the ridge
    peak FLOP/s / peak B/s); "achieved", "peak" and "frac" are on that side."""
    t_mfma = flops / (mfma_peak_tflops * 1e12) if flops else 0.0
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    tf = flops / seconds / 1e12
    gbs = nbytes / seconds / 1e9
    hbm = t_hbm >= t_mfma
    return {
        "kernel": kernel,
        "bound": "hbm" if hbm else "mfma",
        "achieved": round(gbs, 1) if hbm else round(tf, 1),
        "peak": PEAK_HBM_GBS if hbm else mfma_peak_tflops,
        "unit": "GB/s" if hbm else "TFLOP/s",
        "frac": round(gbs / PEAK_HBM_GBS if hbm else tf / mfma_peak_tflops, 4),
        "us_per_launch": round(seconds * 1e6, 2),
        "algorithmic_flop": flops, "algorithmic_bytes": nbytes,
        "intensity_flop_per_byte": round(flops / nbytes, 1),
        "ridge_flop_per_byte": round(mfma_peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "mfma_frac": round(tf / mfma_peak_tflops, 4) if flops else None,
        "algorithmic": how,
    }


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)


def _hip_runtime():
    """The HIP runtime library torch has loaded (the one the library's kernels run on)."""
    import ctypes
    import torch  # noqa: F401  (loads the runtime)
    path = next((l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l), "libamdhip64.so")
    hip = ctypes.CDLL(path)
    P = ctypes.c_void_p
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
    hip.hipEventRecord.argtypes = [P, P]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
    hip.hipEventDestroy.argtypes = [P]
    return hip


class StepMarks:
    """HIP events at fixed points of every timed step, recorded on the current stream
    (the stream the library's kernels are enqueued on): before the gate-up GEMM,
    between the two GEMMs (one event ends the gate-up interval and starts the down
    interval) and after the down GEMM.  Every event recorded between two kernels
    leaves a gap of a few microseconds in the step (kernel trace), so there are as
    few as the two intervals need.  The events are created before the timed loop
    (creating them inside it added tens of microseconds per step) and without the
    system-scope fence (with it, the gap per event was ~5.7 us and the following
    kernel started with the L2 written back)."""

    def __init__(self, steps, marks=3):
        import ctypes
        import torch
        self.hip = _hip_runtime()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.events = []
        for _ in range(steps):
            row = tuple(ctypes.c_void_p() for _ in range(marks))
            for ev in row:
                if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(row)
        self.step = 0

    def mark(self, i):
        if self.hip.hipEventRecord(self.events[self.step][i], self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def next_step(self):
        self.step += 1

    def mean_ms(self, i, j):
        """Mean over the recorded steps of the time from mark i to mark j (call after the
        stream has been synchronized)."""
        import ctypes
        ms = []
        for row in self.events[:self.step]:
            t = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(t), row[i], row[j]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            ms.append(t.value)
        return float(np.mean(ms)) if ms else float("nan")

    def close(self):
        for row in self.events:
            for ev in row:
                self.hip.hipEventDestroy(ev)
        self.events = []


# ----------------------------------------------------------------- prefill

def bench_weight(synth, which, e, n, kk):
    """Expert e's fp32 weights of the benched layer ("gu" or "dn"), N(0, 0.02), drawn on
    the device from a seeded generator (fast for the 32 large experts)."""
    return synth.normal_cuda((31_000 if which == "gu" else 32_000) + e, (n, kk), 0.02)


def setup_prefill(fgg, synth, torch, weight_fn=None):
    """Inputs of the prefill step resident in HBM.  weight_fn(which, e, N, K) gives
    expert e's fp32 weights ("gu" [N_gu, K] or "dn" [N_dn, K_dn]) as a device
    tensor; by default they are drawn on the device (synth.normal_cuda, N(0, 0.02))."""
    cfg = synth.MOE_PREFILL
    T, K, E, k = cfg["T"], cfg["K"], cfg["E"], cfg["k"]
    Ngu, Ndn, Kdn = cfg["N_gu"], cfg["N_dn"], cfg["K_dn"]
    r = synth.moe_prefill_routing()
    ids = torch.from_numpy(r["topk_ids"]).cuda()
    tw = torch.from_numpy(r["topk_w"]).cuda()
    x = torch.from_numpy(synth.moe_prefill_x()).cuda().to(torch.bfloat16)     # layer input, bf16
    gu_q = torch.empty((E, Ngu, K), dtype=torch.uint8, device="cuda")
    gu_s = torch.empty((E, Ngu // 128, K // 128), dtype=torch.float32, device="cuda")
    dn_q = torch.empty((E, Ndn, Kdn), dtype=torch.uint8, device="cuda")
    dn_s = torch.empty((E, Ndn // 128, Kdn // 128), dtype=torch.float32, device="cuda")
    if weight_fn is None:
        def weight_fn(which, e, n, kk):
            return bench_weight(synth, which, e, n, kk)
    for e in range(E):      # offline weight quantization (untimed)
        w = weight_fn("gu", e, Ngu, K)
        fgg.quantize_blockwise(w, fgg.Q_E4M3_128x128, out=gu_q[e], scales=gu_s[e])
        w = weight_fn("dn", e, Ndn, Kdn)
        fgg.quantize_blockwise(w, fgg.Q_E4M3_128x128, out=dn_q[e], scales=dn_s[e])
    del w
    perm = fgg.moe_permute_outputs(T, k, E, 128, K)
    m_cap = perm["m_cap"]
    bufs = dict(
        a2=torch.empty((m_cap, Kdn), dtype=torch.uint8, device="cuda"),
        s2=torch.empty((Kdn // 128, m_cap), dtype=torch.float32, device="cuda"),
        y=torch.empty((m_cap, Ndn), dtype=torch.bfloat16, device="cuda"),
        out=torch.empty((T, Ndn), dtype=torch.bfloat16, device="cuda"),
    )
    useful = 2.0 * int((r["topk_ids"] >= 0).sum()) * (Ngu * K + Ndn * Kdn)
    return dict(cfg=cfg, ids=ids, tw=tw, x=x, gu_q=gu_q, gu_s=gu_s, dn_q=dn_q, dn_s=dn_s, perm=perm,
                bufs=bufs, useful_flops=useful, routing=r)


def prefill_step(fgg, st, marks=None):
    b, p = st["bufs"], st["perm"]
    E = st["cfg"]["E"]
    fgg.moe_permute(st["ids"], E, 128, x=st["x"], out=p)       # 1x128 e4m3 quantization fused in
    if marks:
        marks.mark(0)
    # gate-up grouped GEMM with SiLU(gate)*up and the 1x128 e4m3 requantization in its epilogue
    # (the permute's counts let both GEMMs skip the padding rows of each expert segment)
    fgg.grouped_gemm_silu_quantize(p["a"], p["sa"], st["gu_q"], st["gu_s"], p["offsets"], counts=p["counts"],
                                   out=b["a2"], scales=b["s2"])
    if marks:
        marks.mark(1)
    fgg.grouped_gemm_scaled(b["a2"], b["s2"], st["dn_q"], st["dn_s"], offsets=p["offsets"], masked_m=p["counts"],
                            out=b["y"])
    if marks:
        marks.mark(2)
        marks.next_step()
    fgg.moe_combine(b["y"], p["src_to_row"], st["tw"], out=b["out"])


# ------------------------------------------------------------ secondaries

def time_calls(fn, iters, warmup):
    import torch
    for _ in range(warmup):
        fn(0)
    _sync()
    evs = []
    for i in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        evs.append((a, b))
    _sync()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def bench_decode(fgg, synth, torch, iters=50, copies=3):
    wl = synth.moe_decode(with_weights=False)
    G, M, N, K = wl["G"], wl["M_max"], wl["N"], wl["K"]
    aq, sa = fgg.quantize_blockwise(torch.from_numpy(wl["x"].reshape(G * M, K)).cuda(), fgg.Q_E4M3_1x128)
    sa = sa.reshape(K // 128, G, M).permute(1, 0, 2).contiguous()
    aq = aq.reshape(G, M, K)
    mm = torch.from_numpy(wl["masked_m"]).cuda()
    bqs, bes = [], []
    for c in range(copies):       # distinct copies so that caches cannot serve repeats
        bq = torch.empty((G, N, K // 2), dtype=torch.uint8, device="cuda")
        be = torch.empty((G, N, K // 32), dtype=torch.uint8, device="cuda")
        for e in range(G):
            w = synth.normal_cuda(41_000 + 100 * c + e, (N, K), 0.02)
            fgg.quantize_blockwise(w, fgg.Q_E2M1_E8M0_1x32, out=bq[e], scales=be[e])
        # offline: the weights in the tiled (MFMA operand order) layout the decode kernel streams
        bt, st = fgg.pack_fp4_weights(bq, be)
        del bq, be
        bqs.append(bt)
        bes.append(st)
    d = torch.empty((G, M, N), dtype=torch.bfloat16, device="cuda")
    ms = time_calls(lambda i: fgg.grouped_gemm_scaled(aq, sa, bqs[i % copies], bes[i % copies], masked_m=mm,
                                                      b_qdesc=fgg.Q_E2M1_E8M0_1x32_TILED, out=d, n=N), iters, 5)
    wbytes = G * N * (K // 2) + G * N * (K // 32)
    gbs = wbytes / (ms * 1e-3) / 1e9
    rows = int(wl["masked_m"].sum())
    flops = 2.0 * rows * N * K
    nbytes = wbytes + rows * K * (1 + 4 / 128) + rows * N * 2
    roof = roofline_entry("gemm_masked_fp4_lds_kernel<tiled> (decode masked GEMM)", flops, nbytes, ms * 1e-3,
                          PEAK_FP4_TFLOPS, "2*%d*%d*%d FLOP; bytes = E2M1 weights + E8M0 scales of 32 experts, "
                          "the %d real rows' e4m3 codes + scales, their bf16 outputs" % (rows, N, K, rows))
    return dict(workload="moe_decode G=32 M=1..16 (U) N=4096 K=7168 E2M1+E8M0/32 weights (tiled layout), "
                         "e4m3 1x128 acts",
                us_per_call=round(ms * 1e3, 2), weight_bytes=wbytes, value=round(gbs, 1), unit="GB/s",
                pct_hbm_peak=round(100 * gbs / PEAK_HBM_GBS, 1), roofline=roof)


def bench_dense(fgg, synth, torch, iters=30, copies=3):
    M = N = 4096
    K = 7168
    xq, xs = fgg.quantize_blockwise(synth.normal_cuda(51_000, (M, K)), fgg.Q_E4M3_1x128)
    ws = [fgg.quantize_blockwise(synth.normal_cuda(51_001 + c, (N, K), 0.02), fgg.Q_E4M3_128x128)
          for c in range(copies)]
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ms = time_calls(lambda i: fgg.scaled_gemm(xq, xs, ws[i % copies][0], ws[i % copies][1], out=d), iters, 5)
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return dict(workload="dense 4096x4096x7168 e4m3 1x128 / 128x128", us_per_call=round(ms * 1e3, 2),
                value=round(tf, 1), unit="TFLOP/s", pct_fp8_peak=round(100 * tf / PEAK_FP8_TFLOPS, 1))


def bench_w4a4(fgg, synth, torch, iters=30):
    M, N, K, r = 4096, 3072, 3072, 32
    x = synth.normal_cuda(61_000, (M, K)).to(torch.bfloat16)
    xq, xs = fgg.quantize_blockwise(x, fgg.Q_E2M1_1x16)
    wq, wsc = fgg.quantize_blockwise(synth.normal_cuda(61_001, (N, K), 0.02), fgg.Q_E2M1_1x16)
    ld = synth.normal_cuda(61_002, (K, r), 0.01).to(torch.bfloat16)
    lu = synth.normal_cuda(61_003, (r, N), 0.01).to(torch.bfloat16)
    bias = synth.normal_cuda(61_004, (N,), 0.1).to(torch.bfloat16)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(fgg.scaled_gemm_workspace_bytes(M, N, K, "w4a4", rank=r), dtype=torch.uint8, device="cuda")
    ms = time_calls(lambda i: fgg.scaled_gemm(xq, xs, wq, wsc, qdesc="w4a4", x_bf16=x, l_down=ld, l_up=lu,
                                              bias=bias, out=d, workspace=ws), iters, 5)
    flops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
    tf = flops / (ms * 1e-3) / 1e12
    return dict(workload="w4a4 4096x3072x3072 E2M1 fp32/16 + rank-32 + bias", us_per_call=round(ms * 1e3, 2),
                value=round(tf, 1), unit="TFLOP/s", mfu_fp4_pct=round(100 * tf / PEAK_FP4_TFLOPS, 2))


def bench_down_combine(fgg, st, torch, iters=30):
    """The prefill step's down projection + combine as one call (fgg_moe_down_combine)
    against the two calls it replaces, on the step's own data (alternating, medians)."""
    import numpy as np
    b, p = st["bufs"], st["perm"]
    ws = torch.empty(fgg.moe_down_combine_workspace_bytes(b["a2"].shape[0]), dtype=torch.uint8, device="cuda")
    y2, out2 = torch.empty_like(b["y"]), torch.empty_like(b["out"])

    def two():
        fgg.grouped_gemm_scaled(b["a2"], b["s2"], st["dn_q"], st["dn_s"], offsets=p["offsets"],
                                masked_m=p["counts"], out=b["y"])
        fgg.moe_combine(b["y"], p["src_to_row"], st["tw"], out=b["out"])

    def fused():
        fgg.moe_down_combine(b["a2"], b["s2"], st["dn_q"], st["dn_s"], p["offsets"], p["counts"], p["src_to_row"],
                             p["row_to_src"], st["tw"], y2, out=out2, workspace=ws)

    two()
    fused()
    _sync()
    same = bool(torch.equal(b["out"].view(torch.int16), out2.view(torch.int16)))
    t = ([], [])
    for i in range(2 * iters + 4):
        fn = (two, fused)[i % 2]
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        z.record()
        _sync()
        if i >= 4:
            t[i % 2].append(a.elapsed_time(z) * 1e3)
    return {"workload": "prefill down GEMM (N=7168, K=2048, counts) + combine (T=8192, k=8)",
            "two_calls_us": round(float(np.median(t[0])), 2), "fused_us": round(float(np.median(t[1])), 2),
            "bit_identical": same}


def bench_mxfp4(fgg, synth, torch, iters=30):
    """The W4A4 shape in the MX form (E2M1 with E8M0 per 32 on both operands), the
    same rank-32 branch and bias; the prepared operands are resident, the timed
    call is the low-rank product plus the GEMM."""
    M, N, K, r = 4096, 3072, 3072, 32
    x = synth.normal_cuda(61_000, (M, K)).to(torch.bfloat16)
    xq, xe = fgg.quantize_blockwise(x, fgg.Q_E2M1_E8M0_1x32)
    wq, we = fgg.quantize_blockwise(synth.normal_cuda(61_001, (N, K), 0.02), fgg.Q_E2M1_E8M0_1x32)
    ld = synth.normal_cuda(61_002, (K, r), 0.01).to(torch.bfloat16)
    lu = synth.normal_cuda(61_003, (r, N), 0.01).to(torch.bfloat16)
    bias = synth.normal_cuda(61_004, (N,), 0.1).to(torch.bfloat16)
    d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(fgg.scaled_gemm_workspace_bytes(M, N, K, "mxfp4", rank=r), dtype=torch.uint8, device="cuda")
    ms = time_calls(lambda i: fgg.scaled_gemm(xq, xe, wq, we, qdesc="mxfp4", x_bf16=x, l_down=ld, l_up=lu,
                                              bias=bias, out=d, workspace=ws), iters, 5)
    flops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
    tf = flops / (ms * 1e-3) / 1e12
    nbytes = (M + N) * K // 2 + (M + N) * K // 32 + M * K * 2 + M * N * 2
    return dict(workload="mxfp4 w4a4 4096x3072x3072 E2M1 + E8M0/32 both operands + rank-32 + bias",
                us_per_call=round(ms * 1e3, 2), value=round(tf, 1), unit="TFLOP/s",
                mfu_fp4_pct=round(100 * tf / PEAK_FP4_TFLOPS, 2),
                roofline=roofline_entry("gemm_mxfp4_kernel (+ low-rank prep launch)", flops, nbytes, ms * 1e-3,
                                        PEAK_FP4_TFLOPS, "2MNK + 2Mr(K+N) FLOP; bytes = FP4 codes + E8M0 scales "
                                        "of both operands, the bf16 input of the low-rank branch, bf16 output"))


# ----------------------------------------------------------- CPU baseline

def cpu_baseline(synth, target_s=15.0):
    """The oracle's MoE layer, expert by expert, on the benched layer's routing,
    bf16 input and fp32 weights (the same values the GPU step quantizes: copied
    from the device generator to the host): quantize the expert's tokens (1x128
    e4m3), gate-up GEMM (fp64 per-group formula), SiLU(gate)*up requantized,
    down GEMM, bf16 output and the gate-weighted accumulation into the layer
    output.  Experts are taken largest first until about target_s seconds of
    CPU work; weight quantization is offline (untimed) as on the GPU."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cfg = synth.MOE_PREFILL
    K, Ngu, Ndn, Kdn = cfg["K"], cfg["N_gu"], cfg["N_dn"], cfg["K_dn"]
    r = synth.moe_prefill_routing()
    ids, tw = r["topk_ids"], r["topk_w"]
    counts = np.bincount(ids[ids >= 0], minlength=cfg["E"])
    order = np.argsort(-counts, kind="stable")
    x = synth.to_bf16_values(synth.moe_prefill_x())       # the step's input is bf16
    out = np.zeros((x.shape[0], Ndn))
    flops = 0.0
    elapsed = 0.0
    rows_done = 0
    used = []
    for e in order:
        wq_gu, ws_gu = oracle.quantize_e4m3_blocks(bench_weight(synth, "gu", int(e), Ngu, K).cpu().numpy(), 128, 128)
        wq_dn, ws_dn = oracle.quantize_e4m3_blocks(bench_weight(synth, "dn", int(e), Ndn, Kdn).cpu().numpy(),
                                                   128, 128)
        t0 = time.perf_counter()
        toks, slots = np.nonzero(ids == e)
        aq, sa = oracle.quantize_e4m3_blocks(x[toks], 1, 128)
        seg = np.array([0, len(toks)])
        h = oracle.grouped_gemm_contiguous(aq, sa, wq_gu[None], ws_gu[None], seg)   # fp32 sums fused on the GPU
        a2, s2 = oracle.silu_mul_quantize(h)
        y = oracle.round_bf16(oracle.grouped_gemm_contiguous(a2, s2, wq_dn[None], ws_dn[None], seg))
        out[toks] += tw[toks, slots][:, None] * y
        elapsed += time.perf_counter() - t0
        flops += 2.0 * len(toks) * (Ngu * K + Ndn * Kdn)
        rows_done += len(toks)
        used.append(int(e))
        if elapsed >= target_s:
            break
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle MoE layer (quantize, gate-up, SiLU-requant, down, combine; fp64 per-group GEMM "
                      f"formula) on the {len(used)} largest local experts of the prefill routing: {rows_done} of "
                      f"{int((ids >= 0).sum())} routed rows, {flops / 1e9:.1f} of "
                      f"{2.0 * int((ids >= 0).sum()) * (Ngu * K + Ndn * Kdn) / 1e9:.1f} GFLOP, in {elapsed:.1f} s"}


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks settle within a few tens of steps: with 5 warm-up steps the first timed
    # steps are ~5% slower than from the 50th on (0.667 vs 0.636 ms per step)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (reference dispatch for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU path only (one MI355X); there is no multi-GPU mode: "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import fp4_grouped_gemm_amd as fgg
    import synth

    fgg.load_library()
    dev = torch.cuda.get_device_properties(0)
    st = setup_prefill(fgg, synth, torch)
    _sync()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        _sync()
        dst.copy_(src)           # reads and writes exactly 1 GiB
        _sync()
        del src, dst

    for _ in range(args.warmup):
        prefill_step(fgg, st)
    _sync()
    # the timed steps: nothing but the step's kernels on the stream
    t0 = time.perf_counter()
    for _ in range(args.steps):
        prefill_step(fgg, st)
    _sync()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # the same number of steps again with HIP events between the kernels, for the
    # GEMMs' own durations (each event leaves a gap of a few microseconds in the
    # stream, so these steps are not the ones the step time is taken from)
    marks = StepMarks(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        prefill_step(fgg, st, marks)
    _sync()
    ms_step_marked = (time.perf_counter() - t0) * 1e3 / args.steps
    gu_ms, dn_ms = marks.mean_ms(0, 1), marks.mean_ms(1, 2)
    marks.close()

    useful = st["useful_flops"]
    value = useful / (ms_step * 1e-3) / 1e12
    cfg = st["cfg"]
    n_local = int((st["routing"]["topk_ids"] >= 0).sum())
    gu_flops = 2.0 * n_local * cfg["N_gu"] * cfg["K"]
    dn_flops = 2.0 * n_local * cfg["N_dn"] * cfg["K_dn"]
    gu_tf = gu_flops / (gu_ms * 1e-3) / 1e12
    m_total = int(st["perm"]["offsets"][cfg["E"]].item())
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "moe_prefill: T=8192 tokens, K=7168, 32 local experts of 256, top-8, Zipf(1.1) "
                        "segments padded to 128 (M_total=%d), gate-up N=4096, SiLU*up e4m3 requant, down N=7168 "
                        "K=2048, combine; e4m3 1x128 activations, 128x128 weights, bf16 out" % m_total,
            "global_batch": cfg["T"],
            "parallelism": "single GPU (one expert-parallel shard)",
            "device": dev.name,
        },
        "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "gemm_only": {
            "gate_up_us": round(gu_ms * 1e3, 2), "down_us": round(dn_ms * 1e3, 2),
            "ms_per_step_with_events": round(ms_step_marked, 4),
            "tflops": round((gu_flops + dn_flops) / ((gu_ms + dn_ms) * 1e-3) / 1e12, 1),
            "useful_gflop": round((gu_flops + dn_flops) / 1e9, 1),
        },
    }
    # algorithmic bytes: what a kernel that reads every operand byte and writes every
    # output byte once must move (routed rows only; padding rows carry no data)
    K, Ngu, Ndn, Kdn, E = cfg["K"], cfg["N_gu"], cfg["N_dn"], cfg["K_dn"], cfg["E"]
    I = Ngu // 2
    gu_bytes = (n_local * K * (1 + 4 / 128) + E * Ngu * K * (1 + 4 / (128 * 128)) + n_local * I * (1 + 4 / 128))
    dn_bytes = (n_local * Kdn * (1 + 4 / 128) + E * Ndn * Kdn * (1 + 4 / (128 * 128)) + n_local * Ndn * 2)
    gu_roof = roofline_entry(
        "gemm_fp8_contig_kernel<silu> (gate-up grouped GEMM, SiLU requant epilogue)", gu_flops, gu_bytes,
        gu_ms * 1e-3, PEAK_FP8_TFLOPS,
        "2*%d*%d*%d FLOP; bytes = routed rows' e4m3 codes + 1x128 scales, all experts' gate-up weights + "
        "128x128 scales, requantized output codes + scales" % (n_local, Ngu, K))
    gu_roof["traffic"] = measured_traffic(os.path.dirname(os.path.abspath(__file__)))
    gu_roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, copy-calibrated)"
    result["roofline"] = gu_roof
    result["rooflines"] = {
        "gate_up": gu_roof,
        "down": roofline_entry(
            "gemm_fp8_contig_kernel<plain> (down grouped GEMM)", dn_flops, dn_bytes, dn_ms * 1e-3, PEAK_FP8_TFLOPS,
            "2*%d*%d*%d FLOP; bytes = routed rows' e4m3 codes + scales, all experts' down weights + scales, "
            "bf16 outputs of the routed rows" % (n_local, Ndn, Kdn)),
    }
    if not args.no_secondary:
        dec = bench_decode(fgg, synth, torch)
        result["rooflines"]["decode"] = dec.pop("roofline")
        result["secondary"] = {
            "moe_decode": dec,
            "dense": bench_dense(fgg, synth, torch),
            "w4a4": bench_w4a4(fgg, synth, torch),
        }
        result["secondary"]["moe_down_combine"] = bench_down_combine(fgg, st, torch)
        mx = bench_mxfp4(fgg, synth, torch)
        result["rooflines"]["mxfp4"] = mx.pop("roofline")
        result["secondary"]["mxfp4"] = mx
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
