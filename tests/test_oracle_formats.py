"""Pins for the oracle's codecs: tables against the formats' definitions and
against independent library decoders; encoders against brute force."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            out.append((int(c, 16), float(v)))
    return out


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_e2m1_table_matches_page_values():
    for code, val in _read_pairs("e2m1_values.txt"):
        assert _same(F.E2M1_TABLE[code], val), hex(code)
    mags = sorted(set(np.abs(F.E2M1_TABLE)))
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert F.E2M1_TABLE.max() == 6.0 and F.E2M1_TABLE.min() == -6.0   # range ±6


def test_e4m3_table_golden_and_counts():
    for code, val in _read_pairs("e4m3_values.txt"):
        assert _same(F.E4M3_TABLE[code], val), hex(code)
    finite = np.isfinite(F.E4M3_TABLE)
    assert finite.sum() == 254 and np.isnan(F.E4M3_TABLE).sum() == 2
    assert np.nanmax(F.E4M3_TABLE) == 448.0            # [DeepGEMM] §2.1: max ≈ 448
    pos = F.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # codes ascend with magnitude


def test_e4m3_table_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        assert _same(F.E4M3_TABLE[b], ref[b]), hex(b)


def test_e8m0_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = F.decode_e8m0(np.arange(256))
    for b in range(256):
        assert _same(mine[b], ref[b]), b


def _brute_encode(x, table_pos, sign_bit):
    """Nearest magnitude by exhaustive search, ties to the even code, saturating."""
    a = abs(x)
    if a >= table_pos[-1]:
        c = len(table_pos) - 1
    else:
        best = None
        for c_ in range(len(table_pos)):
            d = abs(table_pos[c_] - a)
            if best is None or d < best[0] or (d == best[0] and c_ % 2 == 0):
                best = (d, c_)
        c = best[1]
    return c | (sign_bit if math.copysign(1.0, x) < 0 else 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_encoder_brute_force_on_all_midpoints(fmt):
    if fmt == "e4m3":
        pos, sign, enc = F.E4M3_TABLE[:0x7F], 0x80, F.encode_e4m3
    else:
        pos, sign, enc = F.E2M1_TABLE[:8], 0x8, F.encode_e2m1
    mids = (pos[1:] + pos[:-1]) / 2
    pts = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                          pos[-1] * np.array([1.0001, 1.5, 10.0, 1e30]), [1e-30, 0.0]])
    pts = np.concatenate([pts, -pts])
    got = enc(pts)
    for x, c in zip(pts, got):
        assert c == _brute_encode(float(x), pos, sign), (fmt, x)


def test_encode_e4m3_matches_torch_rne_in_range():
    g = np.random.default_rng(5)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    x = x[np.abs(x) < 464].astype(np.float32)          # torch's cast gives NaN beyond 464
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.encode_e4m3(x), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_encode_decode_roundtrip(fmt):
    n = 256 if fmt == "e4m3" else 16
    dec = F.decode_e4m3 if fmt == "e4m3" else F.decode_e2m1
    enc = F.encode_e4m3 if fmt == "e4m3" else F.encode_e2m1
    codes = np.arange(n, dtype=np.uint8)
    keep = ~np.isnan(dec(codes))
    assert np.array_equal(enc(dec(codes[keep])), codes[keep])


def test_saturation_and_sign_of_zero():
    assert F.encode_e4m3([1e9, -1e9, 500.0, -0.0, -1e-30]).tolist() == [0x7E, 0xFE, 0x7E, 0x80, 0x80]
    # 5 is the midpoint of 4 (code 6) and 6 (code 7): ties go to the even code
    assert F.encode_e2m1([7.0, 5.0, -5.0, 0.25, 0.75, -0.0]).tolist() == [0x7, 0x6, 0xE, 0x0, 0x2, 0x8]


def test_pack_unpack_e2m1():
    c = np.arange(16, dtype=np.uint8)
    p = F.pack_e2m1x2(c)
    assert p.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(F.unpack_e2m1x2(p), c)


def test_round_bf16_matches_torch_on_fp32_values():
    g = np.random.default_rng(7)
    x = np.concatenate([g.standard_normal(50000) * s for s in (1e-40, 1e-5, 1, 1e5, 1e38)])
    x = np.clip(x, -3e38, 3e38).astype(np.float32)
    ref = torch.from_numpy(x).bfloat16().double().numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_single_rounding_from_float64():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1+2^-7: tie to even -> 1.
    # 1 + 2^-8 + 2^-40 lies above the midpoint: rounds up (a double rounding via fp32
    # would first drop the 2^-40 and then round the tie down).
    v = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 3 * 2.0 ** -8)])
    assert oracle.round_bf16(v).tolist() == [1.0, 1 + 2.0 ** -7, -(1 + 2 * 2.0 ** -7)]
    assert oracle.bf16_bits(np.array([1.0, -2.0])).tolist() == [0x3F80, 0xC000]


# ------------------------------------------------------------- tiled FP4 weights

@pytest.mark.parametrize("G,N,K", [(2, 32, 384), (1, 16, 1024), (3, 48, 640)])
def test_tile_fp4_weights_is_a_permutation_with_padding(G, N, K):
    """The tiled codes are a permutation of the packed codes, the tiled scales
    hold every scale byte once plus 127-padding to whole 16-byte spans, and
    untiling restores both arrays."""
    rng = np.random.default_rng(G * 1000 + N + K)
    b = rng.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)
    s = rng.integers(100, 140, size=(G, N, K // 32), dtype=np.uint8)
    codes, scales = oracle.tile_fp4_weights(b, s)
    nspan = -(-(K // 32) // 16)
    assert codes.size == b.size and scales.size == G * (N // 16) * nspan * 256
    assert np.array_equal(np.sort(codes), np.sort(b.reshape(-1)))
    pad = scales.size - s.size
    assert np.count_nonzero(scales == 127) == np.count_nonzero(s == 127) + pad
    assert np.array_equal(np.sort(scales[scales != 127]), np.sort(s[s != 127]))
    b2, s2 = oracle.untile_fp4_weights(codes, scales, G, N, K)
    assert np.array_equal(b2, b) and np.array_equal(s2, s)


def test_tile_fp4_weights_worked_positions():
    """Worked example of the stated layout: in a [1, 32, 256] weight (2 K blocks of
    64 bytes per row, two 16-row groups), the byte of row 21 (group 1, r = 5) at
    packed position 100 (K block 1, 16-byte chunk c = 2, byte 4) sits in tile
    (nb 1, kb 1) = 3, piece 16·2 + 5 = 37: offset 3·1024 + 37·16 + 4 = 3668.  Its
    scale byte 6 (of 8 per row: span 0) sits at span (nb 1, j 0) = 1, row 5, byte 6:
    offset 256 + 5·16 + 6 = 342; bytes 8..15 of every row's span are padding (127)."""
    b = np.zeros((1, 32, 128), np.uint8)
    s = np.zeros((1, 32, 8), np.uint8)
    b[0, 21, 100] = 0xA5
    s[0, 21, 6] = 0x81
    codes, scales = oracle.tile_fp4_weights(b, s)
    assert np.flatnonzero(codes).tolist() == [3668] and codes[3668] == 0xA5
    assert scales[342] == 0x81
    assert np.count_nonzero(scales == 0x81) == 1
    spans = scales.reshape(2, 16, 16)
    assert np.all(spans[:, :, 8:] == 127) and np.count_nonzero(spans[:, :, :8]) == 1
