"""MoE routing glue: permute into per-expert segments, and the weighted combine
(oracle; test infrastructure).

[DeepGEMM] §5.3: the grouped GEMM is told each group's id and token offsets,
and every expert's rows must be contiguous.  [FP4MoE] §4.2: expert group sizes
are rounded up to a multiple of 128.  [MegaMoE] §1 and §3: the layer ends with
the gate-weighted sum of the selected experts' outputs.
"""

import numpy as np


def moe_permute(topk_ids, num_experts: int, align: int = 128):
    """Stable counting-sort of (token, slot) pairs by expert.

    topk_ids: int [T, k]; ids outside [0, E) are dropped (not routed here).
    Pair p = t·k + j.  Expert e's segment starts at offsets[e]; its length is
    counts[e] rounded up to ``align``; the pairs of expert e fill it in
    increasing p, then padding rows follow.

    Returns dict with offsets [E+1], counts [E], src_to_row [T·k] (-1 =
    dropped), row_to_src [M_cap] (-1 = padding or unused), m_cap.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    E = int(num_experts)
    flat = ids.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(flat == e))
    padded = ((counts + align - 1) // align) * align
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    m_cap = T * k + E * (align - 1)
    src_to_row = np.full(T * k, -1, dtype=np.int64)
    row_to_src = np.full(m_cap, -1, dtype=np.int64)
    for e in range(E):
        pairs = np.flatnonzero(flat == e)               # ascending pair index
        rows = offsets[e] + np.arange(pairs.size)
        src_to_row[pairs] = rows
        row_to_src[rows] = pairs
    return {
        "offsets": offsets.astype(np.int32),
        "counts": counts.astype(np.int32),
        "src_to_row": src_to_row.astype(np.int32),
        "row_to_src": row_to_src.astype(np.int32),
        "m_cap": m_cap,
    }


def gather_permuted(row_to_src, m_total: int, k: int, xq, xs):
    """Rows [0, m_total) of the permuted activation codes and their 1×128
    scales: row r copies token row_to_src[r] // k; padding rows are zero codes
    and zero scales.  xq [T, K] uint8, xs [T, K/128] float32."""
    r2s = np.asarray(row_to_src[:m_total], dtype=np.int64)
    xq = np.asarray(xq)
    xs = np.asarray(xs, dtype=np.float32)
    a = np.zeros((m_total, xq.shape[1]), dtype=np.uint8)
    sa = np.zeros((m_total, xs.shape[1]), dtype=np.float32)
    valid = r2s >= 0
    tok = r2s[valid] // k
    a[valid] = xq[tok]
    sa[valid] = xs[tok]
    return a, sa


def moe_combine(y, src_to_row, topk_w, T: int, k: int) -> np.ndarray:
    """out[t, n] = Σ_j w[t, j] · y[src_to_row[t·k + j], n] over routed slots,
    summed in float64 in increasing j; a token with no routed slot gives 0.
    Returns float64 [T, N] (round with formats.round_bf16 for a bf16 output)."""
    y = np.asarray(y, dtype=np.float64)
    s2r = np.asarray(src_to_row, dtype=np.int64).reshape(T, k)
    w = np.asarray(topk_w, dtype=np.float64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = s2r[:, j]
        ok = rows >= 0
        out[ok] += w[ok, j][:, None] * y[rows[ok]]
    return out
