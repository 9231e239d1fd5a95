"""CPU oracle for the block-scaled FP8/FP4 MoE grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``fp4_grouped_gemm_amd`` and its HIP library) never
imports it, and this package imports nothing from the product path: the two
share no code, tables, constants or helpers.  The seeded input generators live
in ``synth.py`` (no arithmetic of the method there).

Everything here is plain numpy, written for readability, not speed: codecs are
table lookups built from the bit-field definitions, every contraction follows
the per-group formula in float64, and every rounding step is spelled out.

Sources (web pages; cited below by tag and section):

[FP4MoE]   "Blackwell架构下FP4 MoE模型的TFLOPS性能优化" (intelliparadigm.com):
           §3.1 packed FP4 weight block, §3.2 pipeline, §4.2 tuning rules
           (expert group size a multiple of 128).
[W4A4]     "最新GPU架构上W4A4算子的Warp专用化内核实践" (service.ruibaoantu.com):
           §1 the W4A4 operator equation Y = (Q(X)·Q(W)ᵀ) ⊙ scale + L(X) + b,
           §2 MFU definition, §6 the shared-memory budget formula.
[Infra]    "腾讯 AI Infra" interview notes (ningzhengsheng.cn):
           Q "FP4量化是什么" (E2M1 format table: 1-2-1 bits, 16 values, ±6),
           Q "量化矩阵乘的维度和流程" (online quantization flow, scale
           granularity table, per-group quantize/dequantize and the grouped-K
           GEMM formula Y = Σ_g (X[:,g] × W_q[g,:]) × scale_w[g,:]).
[MegaMoE]  Hopper + DeepGEMM MoE article (www.mqxn.cn/news/59821):
           §1 MoE layer = gate, top-k, experts, weighted sum;
           §2.1 fp8_gemm returning C·(A_scale·B_scale); §3 Mega-MoE flow;
           §3.1 fused GEMM + Swish x/(1+e^{-x}); §4.2 e4m3 range check 448.
[DeepGEMM] DeepGEMM FP8 GEMM teardown (bhfrc.com/news/60438):
           §2.1 format table (e4m3: 4 exponent / 3 mantissa bits, max ≈ 448),
           §2.2 fine-grained scaling inside the kernel, §2.3 FP32
           accumulation over all of K, §5.1 alignment and external padding,
           §5.2 scale = max|x| / 448, §5.3 group ids and token offsets, keep
           each expert's rows contiguous, first test: 2 experts × 8 tokens.

Readings of points the pages leave open (used consistently here):
  rounding is round-to-nearest, ties to the even code; overflow saturates to
  the largest finite code; the quotient x/s is rounded to fp32 before
  encoding; an all-zero block gets scale 1; out-of-range expert ids are
  dropped; E8M0 exponents are the smallest power of two with 6·2^e ≥ amax;
  the gate-up output is laid out [gate | up]; the low-rank branch reads the
  unquantized input rounded to bf16; the per-column affine is a bias.

parity unpinned: ``silu_mul`` numerics beyond fp64 recomputation against a
library sigmoid, and the W4A4 low-rank branch beyond brute-force matmul.
"""

from .formats import (  # noqa: F401
    E4M3_TABLE,
    E2M1_TABLE,
    decode_e4m3,
    decode_e2m1,
    decode_e8m0,
    encode_e4m3,
    encode_e2m1,
    round_bf16,
    bf16_bits,
    pack_e2m1x2,
    unpack_e2m1x2,
    tile_fp4_weights,
    untile_fp4_weights,
)
from .quantize import (  # noqa: F401
    quantize_e4m3_blocks,
    quantize_e2m1_fp32_groups,
    quantize_e2m1_e8m0_groups,
    silu_mul,
    silu_mul_quantize,
    e8m0_exponent,
)
from .moe import moe_permute, moe_combine, gather_permuted  # noqa: F401
from .gemm import (  # noqa: F401
    grouped_gemm_contiguous,
    grouped_gemm_masked,
    scaled_gemm_dense,
    w4a4_lowrank_gemm,
    mxfp4_lowrank_gemm,
)
