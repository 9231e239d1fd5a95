"""Block quantizers and the SiLU·up activation (oracle; test infrastructure).

All quantizers follow the per-group quantize rule of [Infra] Q
"量化矩阵乘的维度和流程" (per-group table: every group of contiguous elements
shares one scale; the code is round(x / scale)), with the scale taken from the
block's largest magnitude as in [DeepGEMM] §5.2 (scale = max|x| / 448 for e4m3;
6 plays the role of 448 for E2M1, the format's largest magnitude per [Infra]
Q "FP4量化是什么").

Arithmetic is done in the precision the readings fix: amax is exact, the scale
is the fp32 quotient fl32(amax / fmt_max), the encoded value is the fp32
quotient fl32(x / s), then round-to-nearest-even with saturation.
"""

import numpy as np

from .formats import encode_e2m1, encode_e4m3

E4M3_MAX = np.float32(448.0)
E2M1_MAX = np.float32(6.0)


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    assert x.dtype in (np.float32, np.float64)
    x32 = x.astype(np.float32)
    assert x.dtype == np.float32 or np.array_equal(x32.astype(np.float64), x), \
        "inputs must be exact fp32 values (fp32 or bf16 data)"
    return x32


def _block_view(x32: np.ndarray, br: int, bc: int) -> np.ndarray:
    r, c = x32.shape
    assert r % br == 0 and c % bc == 0, "partial blocks are not part of the method here"
    return x32.reshape(r // br, br, c // bc, bc)


def _fp32_scale(amax: np.ndarray, fmt_max: np.float32) -> np.ndarray:
    s = (amax.astype(np.float32) / fmt_max).astype(np.float32)   # fl32(amax / fmt_max)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_e4m3_blocks(x, block_rows: int, block_cols: int = 128):
    """e4m3 codes with one fp32 scale per [block_rows × block_cols] block.

    block_rows=1   : per-token 1×128 activation groups (scales [R, C/128]).
    block_rows=128 : 128×128 weight blocks (scales [R/128, C/128]).
    Returns (codes uint8 [R, C], scales float32 [R/block_rows, C/block_cols]).
    """
    x32 = _as_f32(x)
    blocks = _block_view(x32, block_rows, block_cols)
    amax = np.abs(blocks).max(axis=(1, 3))                          # exact
    s = _fp32_scale(amax, E4M3_MAX)
    q32 = (blocks / s[:, None, :, None]).astype(np.float32)         # fl32(x / s)
    codes = encode_e4m3(q32).reshape(x32.shape)
    return codes, s


def quantize_e2m1_fp32_groups(x, group: int = 16):
    """E2M1 codes (one per element, unpacked) with one fp32 scale per
    ``group`` contiguous elements along each row: s = fl32(amax / 6)."""
    x32 = _as_f32(x)
    blocks = _block_view(x32, 1, group)
    amax = np.abs(blocks).max(axis=(1, 3))
    s = _fp32_scale(amax, E2M1_MAX)
    q32 = (blocks / s[:, None, :, None]).astype(np.float32)
    codes = encode_e2m1(q32).reshape(x32.shape)
    return codes, s


def e8m0_exponent(amax: float) -> int:
    """Smallest integer e with 6·2^e >= amax (so the block never clips),
    clamped to the E8M0 range [-127, 127]; 0 for an all-zero block."""
    if amax == 0:
        return 0
    e = int(np.ceil(np.log2(amax / 6.0)))
    while 6.0 * 2.0 ** (e - 1) >= amax:    # exact comparisons fix any log2 rounding
        e -= 1
    while 6.0 * 2.0 ** e < amax:
        e += 1
    return max(-127, min(127, e))


def quantize_e2m1_e8m0_groups(x, group: int = 32):
    """E2M1 codes with one E8M0 power-of-two scale per ``group`` elements.

    Returns (codes uint8 [R, C] one nibble each, scale bytes uint8 [R, C/group]).
    The encoded value is x·2^-e, an exact scaling.
    """
    x32 = _as_f32(x)
    blocks = _block_view(x32, 1, group)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float64)
    e = np.vectorize(e8m0_exponent, otypes=[np.int64])(amax)
    scaled = blocks.astype(np.float64) * np.ldexp(1.0, -e)[:, None, :, None]
    codes = encode_e2m1(scaled).reshape(x32.shape)
    return codes, (e + 127).astype(np.uint8)


def silu_mul(h) -> np.ndarray:
    """SiLU(gate)·up over a [R, 2C] gate-up output laid out [gate | up]:
    a = g / (1 + e^-g) · u in float64 ([MegaMoE] §3.1 Swish form)."""
    h = np.asarray(h, dtype=np.float64)
    c = h.shape[1] // 2
    g, u = h[:, :c], h[:, c:]
    return g / (1.0 + np.exp(-g)) * u


def silu_mul_quantize(h, block_cols: int = 128):
    """SiLU(gate)·up, rounded once to fp32, then 1×128 e4m3 quantization."""
    a32 = silu_mul(h).astype(np.float32)
    return quantize_e4m3_blocks(a32, 1, block_cols)
