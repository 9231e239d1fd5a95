"""Pins for the oracle's permute and combine: the hand-worked 2-experts × 8-tokens
case, invariants of a stable padded counting sort, an independent sort, and
special cases of the weighted combine."""

import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    d = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            key, *vals = line.split()
            d[key] = [int(v) for v in vals]
    return d


def test_permute_two_experts_eight_tokens_golden():
    d = _read_kv("permute_2x8.txt")
    T, k, E, align = d["T"][0], d["k"][0], d["E"][0], d["align"][0]
    ids = np.array(d["topk_ids"], dtype=np.int32).reshape(T, k)
    r = oracle.moe_permute(ids, E, align)
    assert r["counts"].tolist() == d["counts"]
    assert r["offsets"].tolist() == d["offsets"]
    assert r["src_to_row"].tolist() == d["src_to_row"]
    assert r["row_to_src"][0:8].tolist() == d["row_to_src_expert0"]
    assert r["row_to_src"][128:136].tolist() == d["row_to_src_expert1"]
    assert np.all(r["row_to_src"][8:128] == -1) and np.all(r["row_to_src"][136:] == -1)


def _check_permute_invariants(ids, E, align, r):
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert r["counts"].tolist() == counts.tolist()
    padded = -(-counts // align) * align
    assert r["offsets"].tolist() == [0] + np.cumsum(padded).tolist()
    s2r, r2s = r["src_to_row"].astype(np.int64), r["row_to_src"].astype(np.int64)
    assert np.all(s2r[~valid] == -1)
    # bijection between routed pairs and non-padding rows
    assert np.array_equal(r2s[s2r[valid]], np.flatnonzero(valid))
    used = r2s >= 0
    assert used.sum() == valid.sum() and np.array_equal(s2r[r2s[used]], np.flatnonzero(used))
    # each row lies inside its expert's segment; rows ascend with pair index (stable)
    off = r["offsets"]
    for e in range(E):
        seg = r2s[off[e]:off[e + 1]]
        body = seg[:counts[e]]
        assert np.all(flat[body] == e) and np.all(np.diff(body) > 0)
        assert np.all(seg[counts[e]:] == -1)
    # an independent stable sort by (expert, pair index)
    order = sorted(np.flatnonzero(valid).tolist(), key=lambda p: (flat[p], p))
    rank = {}
    for p in order:
        e = flat[p]
        rank[e] = rank.get(e, -1) + 1
        assert s2r[p] == off[e] + rank[e]


@pytest.mark.parametrize("seed,T,k,E", [(1, 64, 2, 4), (2, 300, 8, 32), (3, 1000, 6, 17)])
def test_permute_invariants_random(seed, T, k, E):
    g = synth.rng(seed)
    ids = g.integers(-2, E + 2, size=(T, k)).astype(np.int32)     # includes dropped ids
    r = oracle.moe_permute(ids, E, 128)
    _check_permute_invariants(ids, E, 128, r)


def test_permute_moe_prefill_routing():
    ids = synth.moe_prefill_routing()["topk_ids"]
    r = oracle.moe_permute(ids, 32, 128)
    _check_permute_invariants(ids, 32, 128, r)
    assert r["offsets"][-1] == 10112 and r["counts"].sum() == 8192


def test_gather_permuted_rows_and_padding():
    ids = np.array([[1, 0], [0, 2], [2, 1]], dtype=np.int32)
    xq = np.arange(3 * 256, dtype=np.uint8).reshape(3, 256)
    xs = np.arange(6, dtype=np.float32).reshape(3, 2) + 1
    r = oracle.moe_permute(ids, 3, 128)
    a, sa = oracle.gather_permuted(r["row_to_src"], int(r["offsets"][-1]), 2, xq, xs)
    assert a.shape == (384, 256)
    assert np.array_equal(a[0], xq[0]) and np.array_equal(a[1], xq[1])        # expert 0: pairs 1, 2
    assert np.array_equal(a[128], xq[0]) and np.array_equal(a[129], xq[2])    # expert 1: pairs 0, 5
    assert np.array_equal(a[256], xq[1]) and np.array_equal(a[257], xq[2])    # expert 2: pairs 3, 4
    assert np.all(a[2:128] == 0) and np.all(sa[2:128] == 0)
    assert sa[129].tolist() == xs[2].tolist()


def test_combine_special_cases():
    g = synth.rng(21)
    T, k, N = 50, 3, 64
    y = synth.normal(g, (400, N))
    ids = g.integers(-1, 4, size=(T, k)).astype(np.int32)
    r = oracle.moe_permute(ids, 4, 64)
    w = g.random((T, k)).astype(np.float32)
    out = oracle.moe_combine(y, r["src_to_row"], w, T, k)
    # brute force over tokens and slots
    for t in range(T):
        ref = np.zeros(N)
        for j in range(k):
            row = r["src_to_row"][t * k + j]
            if row >= 0:
                ref = ref + float(w[t, j]) * y[row].astype(np.float64)
        np.testing.assert_allclose(out[t], ref, rtol=0, atol=1e-15)
    # tokens with no routed slot are zero
    none = np.all(ids < 0, axis=1)
    assert np.all(out[none] == 0)
    # k = 1 with unit weight is an exact gather
    ids1 = g.integers(0, 4, size=(T, 1)).astype(np.int32)
    r1 = oracle.moe_permute(ids1, 4, 64)
    out1 = oracle.moe_combine(y, r1["src_to_row"], np.ones((T, 1), np.float32), T, 1)
    assert np.array_equal(out1, y[r1["src_to_row"]].astype(np.float64))
    # linear in the weights
    out2 = oracle.moe_combine(y, r["src_to_row"], 2 * w, T, k)
    assert np.array_equal(out2, 2 * out)
