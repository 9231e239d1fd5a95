"""Exact codecs for e4m3, E2M1, E8M0 and bf16 (oracle; test infrastructure).

Decoding is a lookup in a table that is built here from the bit-field
definition of each format; encoding is "nearest representable value, ties to
the even code, saturate to the largest finite magnitude", written as a search
over that same table.

Format facts the tables must reproduce:
  * e4m3 (FP8, OCP "FN" flavour): 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; largest finite value 448; exponent field 15 with mantissa 7 is NaN;
    no infinities.  [DeepGEMM] §2.1 format table (4/3 bits, max ≈ 448).
  * E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; 16 codes,
    magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, range ±6.
    [Infra] Q "FP4量化是什么", FP4 format table.
  * E8M0: an unsigned power of two 2^(b-127); 0xFF is NaN.  (Block-scale
    format of the MX formats; the pages name only the block size per 32.)
  * bf16: the upper 16 bits of an IEEE binary32, 8 significant bits.
"""

import math

import numpy as np


def _e4m3_bits_to_value(b: int) -> float:
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)          # subnormal: 0.m × 2^(1-bias)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)    # normal: 1.m × 2^(e-bias)
    return -mag if s else mag


def _e2m1_bits_to_value(n: int) -> float:
    s = (n >> 3) & 1
    e = (n >> 1) & 0x3
    m = n & 0x1
    if e == 0:
        mag = (m / 2.0) * 2.0 ** (1 - 1)          # subnormal: 0.m × 2^(1-bias)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)    # normal: 1.m × 2^(e-bias)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_bits_to_value(b) for b in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_bits_to_value(n) for n in range(16)], dtype=np.float64)

# Non-negative finite magnitudes in code order; codes 0..n-1 are ascending.
_E4M3_POS = E4M3_TABLE[:0x7F]   # 0x00..0x7E (0x7F is NaN)
_E2M1_POS = E2M1_TABLE[:8]      # 0x0..0x7


def decode_e4m3(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def decode_e8m0(codes) -> np.ndarray:
    b = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def _encode_nearest_even_sat(x, pos_mags: np.ndarray, sign_bit: int) -> np.ndarray:
    """Round each value to the nearest entry of ``pos_mags`` (by magnitude),
    ties to the even code, saturating at the largest entry; the sign bit is
    copied from the input (so -0 and negative underflow keep their sign)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    n = pos_mags.size
    hi = np.searchsorted(pos_mags, a, side="left")       # pos_mags[hi-1] < a <= pos_mags[hi]
    hi = np.clip(hi, 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    d_lo = a - pos_mags[lo]
    d_hi = pos_mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= pos_mags[-1], n - 1, code)      # saturate to the max finite code
    neg = np.signbit(x)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def encode_e4m3(x) -> np.ndarray:
    """fp64/fp32 values -> e4m3 codes (uint8).  NaN inputs give 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    codes = _encode_nearest_even_sat(x, _E4M3_POS, 0x80)
    return np.where(np.isnan(x), np.uint8(0x7F), codes).astype(np.uint8)


def encode_e2m1(x) -> np.ndarray:
    """fp64/fp32 values -> E2M1 codes (uint8 holding one nibble)."""
    return _encode_nearest_even_sat(x, _E2M1_POS, 0x8)


def pack_e2m1x2(codes) -> np.ndarray:
    """[..., K] nibble codes -> [..., K/2] bytes; element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1x2(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), in one
    rounding step, returned as float64.  bf16 keeps 8 significant bits; its
    smallest normal is 2^-126 and below that the spacing is 2^-133.  Values
    beyond the largest finite bf16 (after rounding) become ±inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, p = np.frexp(xf)                      # |x| = f·2^p, f in [0.5, 1)
    p = np.maximum(p, -125)                  # subnormal range shares the 2^-133 spacing
    ulp = np.ldexp(1.0, p - 8)
    r = np.rint(xf / ulp) * ulp              # np.rint rounds half to even
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def bf16_bits(x) -> np.ndarray:
    """Bit pattern (uint16) of values that are already exact bf16 values."""
    v = np.asarray(x, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v, equal_nan=True), "not a bf16 value"
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0) or np.any(np.isnan(v)), "not a bf16 value"
    return (bits >> 16).astype(np.uint16)


# --------------------------------------------------------------- tiled FP4 layout
# [FP4MoE] §2.1 asks for FP4 data aligned to 128-bit boundaries in an interleaved
# storage format, §3.1 for a dedicated packed weight format.  The library's
# interleave (its header's FGG_E2M1X2_TILED) is stated per 16-row group `nb` of
# an expert `g` and per 128-element K block `kb` (64 bytes of a packed row):
#   a 1024-byte tile, whose 16-byte piece number 16·c + r (c = 0..3, r = 0..15) is
#   row 16·nb + r's packed bytes [64·kb + 16·c, 64·kb + 16·c + 16);
# and for the E8M0 scales per span j of 16 scale bytes (4 K blocks):
#   a 256-byte span, whose bytes [16·r, 16·r + 16) are row 16·nb + r's scale
#   bytes [16·j, 16·j + 16), the positions past the row's K/32 bytes holding 127.
# Tiles and spans follow each other in (g, nb, kb) and (g, nb, j) order.

def tile_fp4_weights(b, b_scales):
    """b uint8 [G, N, K/2], b_scales uint8 [G, N, K/32] ->
    (codes uint8 [G·N·K/2], scales uint8 [G·(N/16)·ceil(K/512)·256]), piece by
    piece as stated above."""
    b = np.asarray(b, dtype=np.uint8)
    s = np.asarray(b_scales, dtype=np.uint8)
    G, N, Kh = b.shape
    nkb, nsc = Kh // 64, s.shape[2]
    nspan = -(-nsc // 16)
    assert N % 16 == 0 and Kh % 64 == 0 and s.shape[:2] == (G, N)
    codes = np.empty(G * N * Kh, dtype=np.uint8)
    scales = np.full(G * (N // 16) * nspan * 256, 127, dtype=np.uint8)
    for g in range(G):
        for nb in range(N // 16):
            for kb in range(nkb):
                tile = ((g * (N // 16) + nb) * nkb + kb) * 1024
                for c in range(4):
                    for r in range(16):
                        piece = tile + (16 * c + r) * 16
                        codes[piece:piece + 16] = b[g, 16 * nb + r, 64 * kb + 16 * c:64 * kb + 16 * c + 16]
            for j in range(nspan):
                span = ((g * (N // 16) + nb) * nspan + j) * 256
                for r in range(16):
                    row = s[g, 16 * nb + r, 16 * j:16 * j + 16]
                    scales[span + 16 * r:span + 16 * r + len(row)] = row
    return codes, scales


def untile_fp4_weights(codes, scales, G, N, K):
    """Inverse of tile_fp4_weights: -> (b [G, N, K/2], b_scales [G, N, K/32])."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    scales = np.asarray(scales, dtype=np.uint8).reshape(-1)
    Kh, nsc = K // 2, K // 32
    nkb, nspan = K // 128, -(-nsc // 16)
    b = np.empty((G, N, Kh), dtype=np.uint8)
    s = np.empty((G, N, nsc), dtype=np.uint8)
    for g in range(G):
        for nb in range(N // 16):
            for kb in range(nkb):
                tile = ((g * (N // 16) + nb) * nkb + kb) * 1024
                for c in range(4):
                    for r in range(16):
                        piece = tile + (16 * c + r) * 16
                        b[g, 16 * nb + r, 64 * kb + 16 * c:64 * kb + 16 * c + 16] = codes[piece:piece + 16]
            for j in range(nspan):
                span = ((g * (N // 16) + nb) * nspan + j) * 256
                for r in range(16):
                    n_here = min(16, nsc - 16 * j)
                    s[g, 16 * nb + r, 16 * j:16 * j + n_here] = scales[span + 16 * r:span + 16 * r + n_here]
    return b, s
