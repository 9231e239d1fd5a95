"""FGG_DEBUG: every launch prints one line naming its kernel, problem, grid and
LDS budget (run in a child process, since the flag is read once per process)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys, torch
sys.path.insert(0, %r)
import fp4_grouped_gemm_amd as fgg
dev = "cuda"
x = torch.randn(256, 512, device=dev)
xq, xs = fgg.quantize_blockwise(x, fgg.Q_E4M3_1x128)
w = torch.randn(2, 256, 512, device=dev) * 0.02
bq = torch.stack([fgg.quantize_blockwise(w[e], fgg.Q_E4M3_128x128)[0] for e in range(2)])
sb = torch.stack([fgg.quantize_blockwise(w[e], fgg.Q_E4M3_128x128)[1] for e in range(2)])
ids = torch.randint(0, 2, (256, 1), dtype=torch.int32, device=dev)
p = fgg.moe_permute(ids, 2, 128, x=x)
q, s = fgg.grouped_gemm_silu_quantize(p["a"], p["sa"], bq, sb, p["offsets"])
h = fgg.grouped_gemm_scaled(p["a"], p["sa"], bq, sb, offsets=p["offsets"], masked_m=p["counts"])
out = fgg.moe_combine(h, p["src_to_row"], torch.ones(256, 1, device=dev))
y = fgg.scaled_gemm(xq, xs, bq[0], sb[0])
xq4, xs4 = fgg.quantize_blockwise(x, fgg.Q_E2M1_1x16)
y4 = fgg.scaled_gemm(xq4, xs4, xq4[:128], xs4[:128], qdesc="w4a4")
xq5, xe5 = fgg.quantize_blockwise(x, fgg.Q_E2M1_E8M0_1x32)
ld = (torch.randn(512, 32, device=dev) * 0.01).to(torch.bfloat16)
lu = (torch.randn(32, 128, device=dev) * 0.01).to(torch.bfloat16)
y5 = fgg.scaled_gemm(xq5, xe5, xq5[:128], xe5[:128], qdesc="mxfp4", x_bf16=x.to(torch.bfloat16), l_down=ld, l_up=lu)
torch.cuda.synchronize()
print("script done")
""" % ROOT


def test_debug_trace_names_every_launch():
    env = dict(os.environ, FGG_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[fgg] ")]
    for kernel in ("quant_e4m3_1x128_kernel", "quant_e4m3_128x128_kernel", "permute_hist_kernel",
                   "permute_scatter_kernel", "permute_quantize_kernel", "gemm_fp8_contig_kernel<silu>",
                   "gemm_fp8_contig_kernel<plain>", "combine_kernel", "gemm_fp8_dense_kernel",
                   "quant_e2m1_1x16_kernel", "w4a4_prep_kernel", "w4a4_gemm_kernel",
                   "quant_e2m1_e8m0_1x32_kernel", "w4a4_lowrank_kernel", "gemm_mxfp4_kernel"):
        hits = [l for l in lines if l.startswith(f"[fgg] {kernel}:")]
        assert hits, f"no trace line for {kernel}"
        assert "grid=" in hits[0] and "lds=" in hits[0]
    assert any("counts" in l for l in lines if "contig_kernel<plain>" in l)
