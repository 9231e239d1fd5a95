"""Pins for the oracle's quantizers: invariants fixed by the scale rule, exact
reconstruction cases, the e4m3 range check, and SiLU against library sigmoids."""

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle import formats as F


def _blocks(x, br, bc):
    r, c = x.shape
    return x.reshape(r // br, br, c // bc, bc)


@pytest.mark.parametrize("br", [1, 128])
def test_e4m3_blocks_hit_448_and_stay_in_range(br):
    g = synth.rng(11)
    x = synth.normal(g, (256, 512)) * np.float32(3.0)
    q, s = oracle.quantize_e4m3_blocks(x, br, 128)
    assert s.shape == (256 // br, 4)
    qb = _blocks(q, br, 128)
    # the element with the block's largest magnitude is encoded as ±448
    assert np.all(np.any((qb == 0x7E) | (qb == 0xFE), axis=(1, 3)))
    dq = F.decode_e4m3(q)
    assert not np.isnan(dq).any() and np.abs(dq).max() <= 448.0      # [MegaMoE] §4.2 range check
    amax = np.abs(_blocks(x, br, 128)).max(axis=(1, 3))
    recon = _blocks(dq, br, 128) * s[:, None, :, None]
    assert np.all(np.abs(recon).max(axis=(1, 3)) <= amax * (1 + 2.0 ** -23))


def test_e4m3_reconstruction_error_bound():
    g = synth.rng(12)
    x = synth.normal(g, (64, 1024))
    q, s = oracle.quantize_e4m3_blocks(x, 1, 128)
    dq = F.decode_e4m3(q)
    pos = F.E4M3_TABLE[:0x7F]
    # half the local code spacing at the decoded value, in scaled units (+ fp32 slack)
    idx = np.searchsorted(pos, np.abs(dq))
    up = pos[np.minimum(idx + 1, 0x7E)] - pos[idx]
    down = pos[idx] - pos[np.maximum(idx - 1, 0)]
    half_step = np.maximum(up, down) / 2
    err = np.abs(x / np.repeat(s, 128, axis=1) - dq)
    assert np.all(err <= half_step + 1e-5 * np.abs(dq) + 1e-12)


def test_e4m3_exact_when_block_is_representable():
    # a block whose values are e4m3 values times 2^p with max 448·2^p has scale
    # exactly 2^p and reproduces its codes
    g = synth.rng(13)
    codes = g.integers(0, 0x7F, size=(8, 128)).astype(np.uint8)
    codes |= (g.integers(0, 2, size=codes.shape) * 0x80).astype(np.uint8)
    codes[:, 5] = 0x7E
    p = g.integers(-6, 6, size=(8, 1))
    x = (F.decode_e4m3(codes) * np.ldexp(1.0, p)).astype(np.float32)
    q, s = oracle.quantize_e4m3_blocks(x, 1, 128)
    assert np.array_equal(s[:, 0], np.ldexp(1.0, p[:, 0]).astype(np.float32))
    assert np.array_equal(q, codes)


def test_zero_block_gets_unit_scale():
    x = np.zeros((2, 256), np.float32)
    x[1, 128:] = 1.0
    x[0, 3] = -0.0
    q, s = oracle.quantize_e4m3_blocks(x, 1, 128)
    assert s[1, 1] == np.float32(1.0) / np.float32(448.0)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert q[0, 3] == 0x80 and np.all(q[0, :3] == 0) and np.all(q[1, 128:] == 0x7E)


def test_per_tensor_scale_when_blocks_share_amax():
    # every 1×128 block with the same amax shares one scale, so the per-group
    # quantizer reduces to the per-tensor one of the online flow
    x = synth.normal(synth.rng(14), (16, 256))
    x[:, 0] = 10.0
    x[:, 128] = -10.0
    x = np.clip(x, -10, 10)
    _, s = oracle.quantize_e4m3_blocks(x, 1, 128)
    assert np.all(s == s[0, 0])


def test_e2m1_fp32_groups_invariants():
    x = synth.normal(synth.rng(15), (32, 256))
    q, s = oracle.quantize_e2m1_fp32_groups(x, 16)
    assert s.shape == (32, 16) and q.max() <= 0xF
    qb = _blocks(q, 1, 16)
    assert np.all(np.any((qb & 0x7) == 0x7, axis=(1, 3)))           # ±6 present
    recon = _blocks(F.decode_e2m1(q), 1, 16) * s[:, None, :, None]
    amax = np.abs(_blocks(x, 1, 16)).max(axis=(1, 3))
    assert np.all(np.abs(recon).max(axis=(1, 3)) <= amax * (1 + 2.0 ** -23))
    # error at most one full step of the coarsest E2M1 spacing (2) times the scale
    err = np.abs(_blocks(x, 1, 16) - recon)
    assert np.all(err <= 1.0 * s[:, None, :, None] * (1 + 1e-6))


def test_e2m1_e8m0_groups_invariants():
    x = synth.normal(synth.rng(16), (32, 512), 0.02)
    x[3, 64:96] = 0.0
    q, e = oracle.quantize_e2m1_e8m0_groups(x, 32)
    assert e.shape == (32, 16) and e.dtype == np.uint8
    amax = np.abs(_blocks(x, 1, 32)).max(axis=(1, 3)).astype(np.float64)
    scale = F.decode_e8m0(e)
    nz = amax > 0
    r = amax[nz] / scale[nz]
    assert np.all((r > 3.0) & (r <= 6.0))                           # smallest non-clipping power of 2
    assert e[3, 2] == 127                                 # zero block -> 2^0
    recon = _blocks(F.decode_e2m1(q), 1, 32) * scale[:, None, :, None]
    xb = _blocks(x, 1, 32).astype(np.float64)
    assert np.all(np.abs(xb) / scale[:, None, :, None] <= 6.0)     # never needs saturation
    assert np.all(np.abs(xb - recon) <= 1.0 * scale[:, None, :, None])   # within half the top step


@pytest.mark.parametrize("amax", [6.0, 6.0000001, 3.0, 3.0000002, 0.75, 1e-30, 1e30])
def test_e8m0_exponent_boundaries(amax):
    e = oracle.e8m0_exponent(amax)
    assert 6.0 * 2.0 ** e >= amax and (e == -127 or 6.0 * 2.0 ** (e - 1) < amax)


def test_silu_mul_matches_library_sigmoids():
    h = synth.normal(synth.rng(17), (8, 512)) * np.float32(4.0)
    a = oracle.silu_mul(h)
    g, u = h[:, :256].astype(np.float64), h[:, 256:].astype(np.float64)
    ref1 = g * scipy.special.expit(g) * u
    ref2 = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(a, ref1, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(a, ref2, rtol=1e-14, atol=1e-300)
    # the [gate | up] split: SiLU applies to the first half only
    assert not np.allclose(a, h[:, 256:] * scipy.special.expit(h[:, 256:]) * h[:, :256])
