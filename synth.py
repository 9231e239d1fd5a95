"""Seeded synthetic workloads for the five benchmark shapes.

This module only draws random inputs (numpy PCG64, float32) and routing
tables; it contains none of the quantization or GEMM arithmetic.  Both the
HIP path (tests, bench) and the oracle consume exactly these arrays.

Workloads (sizes and distributions as stated for each):
  tiny_moe     T=64 tokens, E=4 experts, top-2 from softmax of U[0,1) logits,
               K=256, N=512; X ~ N(0,1) fp32, W[e] ~ N(0,0.02) fp32.
  dense        M=N=4096, K=7168; X ~ N(0,1), W ~ N(0,0.02).
  moe_prefill  T=8192, K=7168, 32 local experts out of 256, top-8; local
               tokens per expert follow Zipf(1.1) proportions; gate-up
               N=4096 (K=7168), down N=7168 (K=2048); W ~ N(0,0.02).
  moe_decode   32 experts with U{1..16} tokens each, K=7168, N=4096;
               X ~ N(0,1), W ~ N(0,0.02).
  w4a4         M=4096, N=K=3072; X ~ N(0,1) with 1% of K channels ×10,
               rounded to bf16; W ~ N(0,0.02); rank-32 L_d, L_u ~ N(0,0.01)
               bf16; bias ~ N(0,0.1) bf16.
"""

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round fp32 data to bf16 storage precision (input preparation: the
    workload's bf16 tensors), returned as fp32 arrays holding bf16 values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().float().numpy()


# ---------------------------------------------------------------- routing ---

def softmax_topk_routing(g: np.random.Generator, T: int, E: int, k: int):
    """Gate stand-in: logits ~ U[0,1) [T, E], p = softmax in float64, the k
    largest p per token (ties to the lower expert id), weights = p of the
    selected experts (not renormalized)."""
    logits = g.random((T, E))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -p), axis=1)
    ids = order[:, :k].astype(np.int32)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(np.float32)
    return ids, w


def zipf_counts(total: int, n: int, s: float) -> np.ndarray:
    """Counts proportional to r^-s for ranks r=1..n, summing to ``total``
    (largest-remainder rounding)."""
    wts = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    exact = wts / wts.sum() * total
    c = np.floor(exact).astype(np.int64)
    rem = total - int(c.sum())
    order = np.argsort(-(exact - c), kind="stable")
    c[order[:rem]] += 1
    return c


def zipf_local_routing(g: np.random.Generator, T: int, k: int, E_local: int, E_global: int,
                       s: float = 1.1):
    """One GPU's share of top-k routing over E_global experts, of which
    E_local live here.  Local pairs total T·k·E_local/E_global and follow Zipf
    proportions over experts (ranks assigned by a seeded permutation); each
    expert takes distinct tokens drawn uniformly; a token holds at most k
    local experts.  Slots not routed here hold -1.  Weights are a softmax of
    U[0,1) logits over the k slots, taken at the local slots."""
    total = T * k * E_local // E_global
    counts = zipf_counts(total, E_local, s)
    rank_to_expert = g.permutation(E_local)
    while True:
        per_tok = np.zeros(T, dtype=np.int64)
        chosen = []
        for r in range(E_local):
            toks = g.choice(T, size=int(counts[r]), replace=False)
            per_tok[toks] += 1
            chosen.append(toks)
        if per_tok.max() <= k:
            break
    ids = np.full((T, k), -1, dtype=np.int32)
    fill = np.zeros(T, dtype=np.int64)
    expert_of_rank = rank_to_expert
    # local ids ascending in the first slots of each token
    for e in range(E_local):
        r = int(np.flatnonzero(expert_of_rank == e)[0])
        for t in np.sort(chosen[r]):
            ids[t, fill[t]] = e
            fill[t] += 1
    logits = g.random((T, k))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = np.where(ids >= 0, p, 0.0).astype(np.float32)
    return ids, w


# ------------------------------------------------------------- workloads ---

def tiny_moe(seed: int = 1001):
    g = rng(seed)
    T, E, k, K, N = 64, 4, 2, 256, 512
    ids, w = softmax_topk_routing(g, T, E, k)
    x = normal(g, (T, K))
    wt = normal(g, (E, N, K), 0.02)
    return dict(T=T, E=E, k=k, K=K, N=N, topk_ids=ids, topk_w=w, x=x, w=wt)


def dense(seed: int = 1002, M: int = 4096, N: int = 4096, K: int = 7168):
    g = rng(seed)
    return dict(M=M, N=N, K=K, x=normal(g, (M, K)), w=normal(g, (N, K), 0.02))


MOE_PREFILL = dict(T=8192, K=7168, E=32, E_global=256, k=8, N_gu=4096, N_dn=7168, K_dn=2048)


def moe_prefill_routing(seed: int = 1003, T: int = 8192, k: int = 8, E: int = 32,
                        E_global: int = 256):
    g = rng(seed)
    ids, w = zipf_local_routing(g, T, k, E, E_global)
    return dict(topk_ids=ids, topk_w=w)


def moe_prefill_x(seed: int = 1003, T: int = 8192, K: int = 7168):
    return normal(rng(seed + 100), (T, K))


def moe_prefill_expert_weight(seed: int, which: str, e: int, N: int, K: int):
    """Weight of local expert e ('gu' or 'dn'), drawn from its own stream so
    that experts can be generated one at a time."""
    tag = {"gu": 1, "dn": 2}[which]
    g = rng(seed * 1000003 + tag * 1009 + e)
    return normal(g, (N, K), 0.02)


def moe_decode(seed: int = 1004, G: int = 32, M_max: int = 16, K: int = 7168, N: int = 4096,
               with_weights: bool = True):
    g = rng(seed)
    masked_m = g.integers(1, M_max + 1, size=G).astype(np.int32)
    x = normal(g, (G, M_max, K))
    out = dict(G=G, M_max=M_max, K=K, N=N, masked_m=masked_m, x=x)
    if with_weights:
        out["w"] = normal(g, (G, N, K), 0.02)
    return out


def moe_decode_expert_weight(seed: int, e: int, N: int, K: int):
    g = rng(seed * 1000003 + 3 * 1009 + e)
    return normal(g, (N, K), 0.02)


def w4a4(seed: int = 1005, M: int = 4096, N: int = 3072, K: int = 3072, rank: int = 32):
    g = rng(seed)
    x = normal(g, (M, K))
    n_out = int(round(0.01 * K))
    outliers = g.permutation(K)[:n_out]
    x[:, outliers] *= np.float32(10.0)
    x = to_bf16_values(x)
    w = normal(g, (N, K), 0.02)
    l_down = to_bf16_values(normal(g, (K, rank), 0.01))
    l_up = to_bf16_values(normal(g, (rank, N), 0.01))
    bias = to_bf16_values(normal(g, (N,), 0.1))
    return dict(M=M, N=N, K=K, rank=rank, x=x, w=w, l_down=l_down, l_up=l_up, bias=bias,
                outlier_channels=np.sort(outliers))


def normal_cuda(seed: int, shape, std: float = 1.0, device: str = "cuda"):
    """N(0, std) fp32 drawn on the device from torch's seeded generator (used for
    the large benchmark weight stacks, which are too slow to draw on the host)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x
