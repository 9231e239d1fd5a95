"""fgg_moe_permute_quantize_noalloc (the entry point for callers that cannot
allocate: its histogram scratch is the library's static device array) against
fgg_moe_permute_quantize with a caller workspace: every output bit for bit, on
two calls in a row, the second smaller, both into buffers pre-filled with
garbage; and the host-side rejection of a problem beyond the scratch."""

import ctypes

import numpy as np
import pytest
import torch

import fp4_grouped_gemm_amd as fgg
import synth
from _util import cuda

MAX_HIST_ENTRIES = (2 * 1024 * 1024 - 256) // 4       # ceil(T·k / 256) · E


def _case(seed, T, k, E, K):
    g = synth.rng(seed)
    ids = g.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    x = synth.to_bf16_values(synth.normal(g, (T, K)))
    return cuda(ids), cuda(x, torch.bfloat16)


def _filled_outputs(T, k, E, K):
    out = fgg.moe_permute_outputs(T, k, E, 128, K)
    for key in ("offsets", "counts", "src_to_row", "row_to_src"):
        out[key].fill_(-77)
    out["a"].fill_(0xCD)
    out["sa"].fill_(-9.0)
    return out


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point_twice_second_smaller():
    for (seed, T, k, E, K) in [(11, 8192, 8, 32, 1024), (12, 777, 3, 5, 640)]:
        ids, x = _case(seed, T, k, E, K)
        want = fgg.moe_permute(ids, E, 128, x=x, out=_filled_outputs(T, k, E, K))
        got = fgg.moe_permute_quantize_noalloc(ids, E, x, _filled_outputs(T, k, E, K))
        torch.cuda.synchronize()
        for key in ("offsets", "counts", "src_to_row", "row_to_src", "a", "sa"):
            assert torch.equal(got[key], want[key]), (seed, key)


def test_noalloc_rejects_problems_beyond_its_scratch():
    lib = fgg.load_library()
    P = ctypes.c_void_p
    good = P(4096)
    E = 1024
    T_ok = (MAX_HIST_ENTRIES // E) * 256               # exactly the largest permute the scratch holds
    T_big = T_ok + 256
    args = lambda T: (good, T, 1, E, 128, good, fgg.FGG_BF16, 128, 128, good, good, good, good, good, good,
                      T + E * 127, None)
    assert lib.fgg_moe_permute_quantize_noalloc(*args(T_big)) == 2        # FGG_ERR_UNSUPPORTED, nothing launched
