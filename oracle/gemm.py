"""Block-scaled grouped GEMM, dense GEMM and W4A4 (oracle; test infrastructure).

The contraction is the per-group formula of [Infra] Q "量化矩阵乘的维度和流程"
(grouped-K GEMM: Y = Σ_g (X[:, g] × W_q[g, :]) × scale_w[g, :]), extended with
the activation's own per-token group scale, as in the online flow of the same
answer (Y = Y_acc × scale_x × scale_w) and [MegaMoE] §2.1 (C·(A_scale·B_scale)):

    Y[r, n] = Σ_kb  s_a[r, kb] · s_b[n, kb] · Σ_{k in block kb} dec(A[r, k]) · dec(B[n, k])

B is stored [G, N, K] (K contiguous), i.e. the Q(W)ᵀ orientation of the W4A4
equation in [W4A4] §1.  Scales multiply each K-block's partial sum inside the
K loop, and the sum runs over all of K in a wide accumulator ([DeepGEMM] §2.2,
§2.3); here that accumulator is float64.

Each e4m3 × e4m3 block sum is exact in float64 (products are multiples of
2^-18 below 2^17.6; 128 of them need < 53 bits), as is the fp32 × fp32 scale
product; the only float64 rounding is in the final multiply-adds.

Outputs are float64; a bf16 result is formats.round_bf16 of it.
"""

import numpy as np

from .formats import decode_e2m1, decode_e4m3, decode_e8m0, unpack_e2m1x2


def _b_block_e4m3(b_codes_g, sb_g, kb, bk=128):
    """Decoded B columns of K-block kb and the per-column block scale."""
    ks = slice(kb * bk, (kb + 1) * bk)
    bd = decode_e4m3(b_codes_g[:, ks])                          # [N, 128]
    n = b_codes_g.shape[0]
    sbn = np.asarray(sb_g, dtype=np.float64)[np.arange(n) // 128, kb]   # 128×128 blocks
    return bd, sbn


def _b_block_e2m1_e8m0(b_packed_g, be_g, kb, bk=128):
    """Decoded and E8M0-scaled (exactly, powers of two) B values of K-block kb."""
    ks = slice(kb * bk, (kb + 1) * bk)
    codes = unpack_e2m1x2(b_packed_g)[:, ks]
    scale32 = decode_e8m0(be_g)[:, kb * bk // 32:(kb + 1) * bk // 32]   # [N, 4]
    bd = decode_e2m1(codes) * np.repeat(scale32, 32, axis=1)
    return bd, np.ones(b_packed_g.shape[0])


def _rows_times_b(a_codes, sa, b_block_fn, K, bk=128):
    """Σ_kb s_a[:, kb] ⊙ (dec(A_kb) @ B_kbᵀ) ⊙ s_b[:, kb] for one group."""
    a_codes = np.asarray(a_codes)
    sa = np.asarray(sa, dtype=np.float64)
    out = None
    for kb in range(K // bk):
        ad = decode_e4m3(a_codes[:, kb * bk:(kb + 1) * bk])      # [R, 128]
        bd, sbn = b_block_fn(kb)
        part = (ad @ bd.T) * sa[:, kb:kb + 1] * sbn[None, :]
        out = part if out is None else out + part
    return out


def grouped_gemm_contiguous(a_codes, sa, b_codes, sb, offsets, rows=None):
    """Contiguous (prefill) layout: rows [offsets[g], offsets[g+1]) of A use
    expert g.  a_codes uint8 [M, K] e4m3; sa float32 [M, K/128] (1×128);
    b_codes uint8 [G, N, K] e4m3; sb float32 [G, N/128, K/128] (128×128).
    Rows outside [0, offsets[G]) are not computed (NaN in the result).
    ``rows`` (optional) restricts the computation to those row indices."""
    a_codes = np.asarray(a_codes)
    offsets = np.asarray(offsets, dtype=np.int64)
    G, N, K = b_codes.shape
    M = a_codes.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.full((rows.size, N), np.nan)
    grp = np.searchsorted(offsets, rows, side="right") - 1
    for g in range(G):
        sel = np.flatnonzero((grp == g) & (rows < offsets[G]))
        if sel.size == 0:
            continue
        r = rows[sel]
        y[sel] = _rows_times_b(a_codes[r], np.asarray(sa)[r],
                               lambda kb, g=g: _b_block_e4m3(b_codes[g], sb[g], kb), K)
    return y


def scaled_gemm_dense(a_codes, sa, b_codes, sb):
    """The one-group case: B [N, K], sb [N/128, K/128]."""
    M = np.asarray(a_codes).shape[0]
    return grouped_gemm_contiguous(a_codes, sa, np.asarray(b_codes)[None],
                                   np.asarray(sb)[None], np.array([0, M]))


def grouped_gemm_masked(a_codes, sa, b, b_scales, masked_m, b_format="e2m1_e8m0"):
    """Masked (decode) layout: for each group g only rows m < masked_m[g] are
    computed; the others are NaN in the result.

    a_codes uint8 [G, M, K] e4m3 with sa float32 [G, M, K/128] (1×128).
    b_format "e2m1_e8m0": b uint8 [G, N, K/2] packed E2M1 (element 2i in the
      low nibble), b_scales uint8 [G, N, K/32] E8M0.
    b_format "e4m3": b uint8 [G, N, K], b_scales float32 [G, N/128, K/128].
    """
    a_codes = np.asarray(a_codes)
    G, M, K = a_codes.shape
    N = b.shape[1]
    y = np.full((G, M, N), np.nan)
    for g in range(G):
        m = int(masked_m[g])
        if m <= 0:
            continue
        if b_format == "e2m1_e8m0":
            fn = lambda kb, g=g: _b_block_e2m1_e8m0(b[g], b_scales[g], kb)  # noqa: E731
        else:
            fn = lambda kb, g=g: _b_block_e4m3(b[g], b_scales[g], kb)  # noqa: E731
        y[g, :m] = _rows_times_b(a_codes[g, :m], np.asarray(sa)[g, :m], fn, K)
    return y


def w4a4_lowrank_gemm(qx, sx, qw, sw, x_bf16=None, l_down=None, l_up=None, bias=None,
                      group=16):
    """[W4A4] §1: Y = (Q(X)·Q(W)ᵀ) ⊙ scale + L(X) + b.

    qx uint8 [M, K] E2M1 codes (one per byte, unpacked) with sx float32
    [M, K/16]; qw uint8 [N, K] with sw float32 [N, K/16].  ⊙ scale is the
    per-16 group scale pair applied inside the K sum.  L(X) = (X_bf16 · L_d) ·
    L_u with L_d [K, r], L_u [r, N], evaluated in float64; b [N]."""
    qx = np.asarray(qx)
    qw = np.asarray(qw)
    M, K = qx.shape
    sx = np.asarray(sx, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    y = np.zeros((M, qw.shape[0]))
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        y += (decode_e2m1(qx[:, ks]) @ decode_e2m1(qw[:, ks]).T) * sx[:, g:g + 1] * sw[None, :, g]
    if l_down is not None:
        xd = np.asarray(x_bf16, dtype=np.float64)
        y += (xd @ np.asarray(l_down, dtype=np.float64)) @ np.asarray(l_up, dtype=np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y


def mxfp4_lowrank_gemm(qx, ex, qw, ew, x_bf16=None, l_down=None, l_up=None, bias=None, group=32):
    """The [W4A4] §1 operator Y = (Q(X)·Q(W)ᵀ) ⊙ scale + L(X) + b with Q in the MX
    form: E2M1 codes and one E8M0 power-of-two scale per 32 elements along K on
    both operands (the per-32 E8M0 block of the decode weights, here on the
    activations too), so that ⊙ scale is the pair 2^(ex-127)·2^(ew-127) applied to
    each 32-element partial sum:

        Y[m, n] = Σ_g  2^(ex[m,g]-127) · 2^(ew[n,g]-127) · Σ_{k in g} dec(qx[m,k]) · dec(qw[n,k])
                  + (X_bf16 · L_d)[m, :] · L_u[:, n] + b[n]

    qx uint8 [M, K] E2M1 codes (one per byte, unpacked) with ex uint8 [M, K/32];
    qw uint8 [N, K] with ew uint8 [N, K/32].  Every partial sum and its power-of-two
    scaling is exact in float64; the low-rank and bias terms are those of
    w4a4_lowrank_gemm."""
    qx = np.asarray(qx)
    qw = np.asarray(qw)
    M, K = qx.shape
    sx = decode_e8m0(ex)                                  # [M, K/32] powers of two
    sw = decode_e8m0(ew)
    y = np.zeros((M, qw.shape[0]))
    for g in range(K // group):
        ks = slice(g * group, (g + 1) * group)
        y += (decode_e2m1(qx[:, ks]) @ decode_e2m1(qw[:, ks]).T) * sx[:, g:g + 1] * sw[None, :, g]
    if l_down is not None:
        xd = np.asarray(x_bf16, dtype=np.float64)
        y += (xd @ np.asarray(l_down, dtype=np.float64)) @ np.asarray(l_up, dtype=np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y
