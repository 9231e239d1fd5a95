"""Python binding of libfgg.so (block-scaled FP8/FP4 MoE grouped GEMM for MI355X).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.  The
names follow the C ABI in ``include/fgg.h``, which documents layouts, formats
and error behaviour.  There is no fallback path: if the library is missing or
the device is not gfx950, calls raise.
"""

import ctypes
import os

import torch

__all__ = [
    "FggError", "load_library", "library_path",
    "Q_E4M3_1x128", "Q_E4M3_128x128", "Q_E2M1_1x16", "Q_E2M1_E8M0_1x32", "Q_E2M1_E8M0_1x32_TILED",
    "quantize_blockwise", "moe_permute", "moe_permute_outputs", "moe_permute_workspace_bytes",
    "moe_permute_quantize_noalloc", "grouped_gemm_scaled", "grouped_gemm_silu_quantize", "pack_fp4_weights",
    "scaled_gemm", "moe_combine", "set_num_cus", "kernel_table", "kernel_compiled_lds",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfgg.so")

FGG_F32, FGG_BF16, FGG_E4M3, FGG_E2M1X2, FGG_E8M0, FGG_E2M1X2_TILED = 0, 1, 2, 3, 4, 5
FGG_ACT_NONE, FGG_ACT_SILU_MUL = 0, 1
FGG_LAYOUT_CONTIGUOUS, FGG_LAYOUT_MASKED = 0, 1
_STATUS = {0: "FGG_OK", 1: "FGG_ERR_INVALID_VALUE", 2: "FGG_ERR_UNSUPPORTED", 3: "FGG_ERR_HIP"}


class FggError(RuntimeError):
    def __init__(self, fn, status, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        extra = f" (hipError {hip_error})" if status == 3 else ""
        super().__init__(f"{fn}: {_STATUS.get(status, status)}{extra}")


class QDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_int32), ("scale", ctypes.c_int32),
                ("block_rows", ctypes.c_int32), ("block_k", ctypes.c_int32)]


class KernelInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("entry", ctypes.c_char_p), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("stage_bytes", ctypes.c_int32), ("other_bytes", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32)]


class Epilogue(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("l_down", ctypes.c_void_p), ("l_up", ctypes.c_void_p),
                ("rank", ctypes.c_int32), ("bias", ctypes.c_void_p)]


Q_E4M3_1x128 = (FGG_E4M3, FGG_F32, 1, 128)
Q_E4M3_128x128 = (FGG_E4M3, FGG_F32, 128, 128)
Q_E2M1_1x16 = (FGG_E2M1X2, FGG_F32, 1, 16)
Q_E2M1_E8M0_1x32 = (FGG_E2M1X2, FGG_E8M0, 1, 32)
Q_E2M1_E8M0_1x32_TILED = (FGG_E2M1X2_TILED, FGG_E8M0, 1, 32)   # masked-GEMM weights from pack_fp4_weights

_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfgg.so once and declare its signatures.  Raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m fp4_grouped_gemm_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "fgg_status_string": ([I32], ctypes.c_char_p),
        "fgg_last_hip_error": ([], I32),
        "fgg_set_num_cus": ([ctypes.c_int], I32),
        "fgg_kernel_count": ([], I32),
        "fgg_kernel_info_get": ([I32, ctypes.POINTER(KernelInfo)], I32),
        "fgg_kernel_compiled_lds": ([I32, ctypes.POINTER(I64)], I32),
        "fgg_quantize_blockwise": ([P, I32, I64, I64, I64, I32, QDesc, P, P, P, P], I32),
        "fgg_moe_permute_workspace": ([I64, I32, I32, ctypes.POINTER(SZ)], I32),
        "fgg_moe_permute": ([P, I64, I32, I32, I32, P, P, I64, P, P, P, P, P, P, I64, P, SZ, P], I32),
        "fgg_moe_permute_quantize": ([P, I64, I32, I32, I32, P, I32, I64, I64, P, P, P, P, P, P, I64, P, SZ, P], I32),
        "fgg_moe_permute_quantize_noalloc": ([P, I64, I32, I32, I32, P, I32, I64, I64, P, P, P, P, P, P, I64, P], I32),
        "fgg_grouped_gemm_scaled": ([I32, I32, I64, I64, I64, P, P, QDesc, P, P, QDesc, P, P, P, I64, P], I32),
        "fgg_grouped_gemm_silu_quantize": ([I32, I64, I64, I64, P, P, QDesc, P, P, QDesc, P, P, P, P, P], I32),
        "fgg_scaled_gemm_workspace": ([I64, I64, I64, QDesc, QDesc, ctypes.POINTER(Epilogue), ctypes.POINTER(SZ)], I32),
        "fgg_scaled_gemm": ([I64, I64, I64, P, P, QDesc, P, P, QDesc, ctypes.POINTER(Epilogue), P, I64, P, SZ, P], I32),
        "fgg_moe_combine": ([P, I64, P, P, I64, I32, I64, P, I64, P], I32),
        "fgg_moe_down_combine_workspace": ([I64, ctypes.POINTER(SZ)], I32),
        "fgg_moe_down_combine": ([I32, I64, I64, I64, P, P, QDesc, P, P, QDesc, P, P, P, P, P, I64, I32, P, I64, P, SZ,
                                  P, I64, P], I32),
        "fgg_pack_fp4_weights_bytes": ([I32, I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I32),
        "fgg_pack_fp4_weights": ([P, P, I32, I64, I64, P, P, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(fn_name, status):
    if status != 0:
        lib = load_library()
        raise FggError(fn_name, status, lib.fgg_last_hip_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _q(desc):
    return QDesc(*desc)


def set_num_cus(n: int) -> None:
    _check("fgg_set_num_cus", load_library().fgg_set_num_cus(int(n)))


def kernel_table():
    """Every kernel of the library with its tile and LDS budget (fgg_kernel_info_get)."""
    lib = load_library()
    out = []
    for i in range(lib.fgg_kernel_count()):
        ki = KernelInfo()
        _check("fgg_kernel_info_get", lib.fgg_kernel_info_get(i, ctypes.byref(ki)))
        d = {f: getattr(ki, f) for f, _ in KernelInfo._fields_}
        d["kernel"] = d["kernel"].decode()
        d["entry"] = d["entry"].decode()
        out.append(d)
    return out


def kernel_compiled_lds(i: int) -> int:
    """Static LDS bytes of kernel i as compiled (asks the HIP runtime; needs the GPU)."""
    n = ctypes.c_int64(0)
    _check("fgg_kernel_compiled_lds", load_library().fgg_kernel_compiled_lds(int(i), ctypes.byref(n)))
    return n.value


# ------------------------------------------------------------------ quantize

def quantize_blockwise(x: torch.Tensor, qdesc=Q_E4M3_1x128, silu_mul: bool = False, out=None, scales=None,
                       rows_dev=None):
    """Quantize a [rows, cols] fp32/bf16 tensor (rows may have a larger stride).

    With silu_mul=True the input has 2·cols columns laid out [gate | up].
    rows_dev (int32 device tensor, one element) limits the rows processed to
    min(rows, rows_dev[0]) without a host synchronization.
    Returns (codes, scales) in the layouts of include/fgg.h:
      Q_E4M3_1x128:     codes uint8 [rows, cols],   scales f32 [cols/128, rows]
      Q_E4M3_128x128:   codes uint8 [rows, cols],   scales f32 [rows/128, cols/128]
      Q_E2M1_1x16:      codes uint8 [rows, cols/2], scales f32 [rows, cols/16]
      Q_E2M1_E8M0_1x32: codes uint8 [rows, cols/2], scales u8  [rows, cols/32]
    """
    assert x.dim() == 2 and x.dtype in (torch.float32, torch.bfloat16) and x.stride(1) == 1
    rows, width = x.shape
    cols = width // 2 if silu_mul else width
    data, sdt, br, bk = qdesc
    dev = x.device
    if out is None:
        out = torch.empty((rows, cols if data == FGG_E4M3 else cols // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        if qdesc == Q_E4M3_1x128:
            shape = (cols // 128, rows)
        elif qdesc == Q_E4M3_128x128:
            shape = (rows // 128, cols // 128)
        else:
            shape = (rows, cols // bk)
        scales = torch.empty(shape, dtype=torch.uint8 if sdt == FGG_E8M0 else torch.float32, device=dev)
    xdt = FGG_F32 if x.dtype == torch.float32 else FGG_BF16
    st = load_library().fgg_quantize_blockwise(
        _ptr(x), xdt, rows, cols, x.stride(0), FGG_ACT_SILU_MUL if silu_mul else FGG_ACT_NONE,
        _q(qdesc), _ptr(rows_dev), _ptr(out), _ptr(scales), _stream(dev))
    _check("fgg_quantize_blockwise", st)
    return out, scales


# ------------------------------------------------------------------- permute

def moe_permute_workspace_bytes(T: int, k: int, E: int) -> int:
    n = ctypes.c_size_t(0)
    _check("fgg_moe_permute_workspace", load_library().fgg_moe_permute_workspace(T, k, E, ctypes.byref(n)))
    return n.value


def moe_permute_outputs(T: int, k: int, E: int, align: int = 128, K: int = 0, m_cap=None, device="cuda"):
    """Allocate the output buffers of moe_permute (for reuse across calls)."""
    if m_cap is None:
        m_cap = T * k + E * (align - 1)
    out = dict(
        offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
        counts=torch.empty(E, dtype=torch.int32, device=device),
        src_to_row=torch.empty(max(T * k, 1), dtype=torch.int32, device=device),
        row_to_src=torch.empty(max(m_cap, 1), dtype=torch.int32, device=device),
        a=None, sa=None, m_cap=m_cap,
        workspace=torch.empty(max(moe_permute_workspace_bytes(T, k, E), 1), dtype=torch.uint8, device=device))
    if K:
        out["a"] = torch.empty((max(m_cap, 1), K), dtype=torch.uint8, device=device)
        out["sa"] = torch.empty((K // 128, max(m_cap, 1)), dtype=torch.float32, device=device)
    return out


def moe_permute(topk_ids: torch.Tensor, num_experts: int, align: int = 128, xq=None, xs=None,
                m_cap=None, workspace=None, out=None, x=None):
    """Stable padded permute.  topk_ids int32 [T, k] on the device.  With xq
    (uint8 [T, K]) and xs (f32 [K/128, T]) the permuted codes/scales are
    gathered too.  With x (bf16 or f32 [T, K], unit column stride) instead,
    the 1x128 e4m3 quantization is fused into the gather
    (fgg_moe_permute_quantize; same outputs as quantizing first).  Returns a
    dict of device tensors (see include/fgg.h); ``out`` (from
    moe_permute_outputs) is filled instead of allocating."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2 and topk_ids.is_contiguous()
    T, k = topk_ids.shape
    E = int(num_experts)
    dev = topk_ids.device
    if x is not None:
        assert xq is None and x.dim() == 2 and x.shape[0] == T and x.stride(1) == 1
        assert x.dtype in (torch.bfloat16, torch.float32)
        K = x.shape[1]
        if out is None:
            out = moe_permute_outputs(T, k, E, align, K, m_cap, dev)
        assert out["a"] is not None and out["a"].shape[1] == K
        if workspace is None:
            workspace = out["workspace"]
        st = load_library().fgg_moe_permute_quantize(
            _ptr(topk_ids), T, k, E, align, _ptr(x), FGG_BF16 if x.dtype == torch.bfloat16 else FGG_F32, K,
            x.stride(0), _ptr(out["offsets"]), _ptr(out["counts"]), _ptr(out["src_to_row"]),
            _ptr(out["row_to_src"]), _ptr(out["a"]), _ptr(out["sa"]), out["m_cap"], _ptr(workspace),
            workspace.numel(), _stream(dev))
        _check("fgg_moe_permute_quantize", st)
        m = out["m_cap"]
        return dict(offsets=out["offsets"], counts=out["counts"], src_to_row=out["src_to_row"][:T * k],
                    row_to_src=out["row_to_src"][:m], a=out["a"], sa=out["sa"], m_cap=m)
    K = 0 if xq is None else xq.shape[1]
    if out is None:
        out = moe_permute_outputs(T, k, E, align, K, m_cap, dev)
    m_cap = out["m_cap"]
    offsets, counts, s2r, r2s = out["offsets"], out["counts"], out["src_to_row"], out["row_to_src"]
    a_out, sa_out = out["a"], out["sa"]
    if xq is not None:
        assert xq.dtype == torch.uint8 and xq.is_contiguous() and xs.is_contiguous()
        assert a_out is not None and a_out.shape[1] == K
    if workspace is None:
        workspace = out["workspace"]
    st = load_library().fgg_moe_permute(
        _ptr(topk_ids), T, k, E, align, _ptr(xq), _ptr(xs), K, _ptr(offsets), _ptr(counts), _ptr(s2r),
        _ptr(r2s), _ptr(a_out), _ptr(sa_out), m_cap, _ptr(workspace), workspace.numel(), _stream(dev))
    _check("fgg_moe_permute", st)
    return dict(offsets=offsets, counts=counts, src_to_row=s2r[:T * k], row_to_src=r2s[:m_cap], a=a_out,
                sa=sa_out, m_cap=m_cap)


def moe_permute_quantize_noalloc(topk_ids: torch.Tensor, num_experts: int, x: torch.Tensor, out, align: int = 128):
    """fgg_moe_permute_quantize_noalloc: the fused permute-quantize with the library's
    static device scratch instead of a workspace (for callers that cannot allocate).
    ``out`` (from moe_permute_outputs) receives every output; its workspace is unused."""
    assert topk_ids.dtype == torch.int32 and topk_ids.dim() == 2 and topk_ids.is_contiguous()
    assert x.dim() == 2 and x.stride(1) == 1 and x.dtype in (torch.bfloat16, torch.float32)
    T, k = topk_ids.shape
    K = x.shape[1]
    assert out["a"] is not None and out["a"].shape[1] == K
    st = load_library().fgg_moe_permute_quantize_noalloc(
        _ptr(topk_ids), T, k, int(num_experts), align, _ptr(x), FGG_BF16 if x.dtype == torch.bfloat16 else FGG_F32,
        K, x.stride(0), _ptr(out["offsets"]), _ptr(out["counts"]), _ptr(out["src_to_row"]), _ptr(out["row_to_src"]),
        _ptr(out["a"]), _ptr(out["sa"]), out["m_cap"], _stream(topk_ids.device))
    _check("fgg_moe_permute_quantize_noalloc", st)
    m = out["m_cap"]
    return dict(offsets=out["offsets"], counts=out["counts"], src_to_row=out["src_to_row"][:T * k],
                row_to_src=out["row_to_src"][:m], a=out["a"], sa=out["sa"], m_cap=m)


# --------------------------------------------------------------------- GEMMs

def grouped_gemm_scaled(a, a_scales, b, b_scales, offsets=None, masked_m=None,
                        b_qdesc=Q_E4M3_128x128, out=None, n=None):
    """Contiguous layout when ``offsets`` is given (a [M, K], a_scales [K/128, M],
    b [G, N, K], b_scales [G, N/128, K/128]); masked layout when ``masked_m``
    is given (a [G, M, K], a_scales [G, K/128, M], b [G, N, K/2] with E8M0
    scales [G, N, K/32] for Q_E2M1_E8M0_1x32, or e4m3 as above).  With
    ``offsets``, an optional ``masked_m`` gives each group's real row count
    (the permute's counts): the padding rows past it are not written.
    With Q_E2M1_E8M0_1x32_TILED (weights from pack_fp4_weights) ``n`` gives N.
    Returns bf16 [M, N] or [G, M, N]."""
    G = b.shape[0]
    N = int(n) if n is not None else b.shape[1]
    dev = a.device
    if offsets is not None:
        M, K = a.shape
        layout = FGG_LAYOUT_CONTIGUOUS
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    else:
        _, M, K = a.shape
        layout = FGG_LAYOUT_MASKED
        if out is None:
            out = torch.empty((G, M, N), dtype=torch.bfloat16, device=dev)
    for t in (a, a_scales, b, b_scales):
        assert t.is_contiguous()
    st = load_library().fgg_grouped_gemm_scaled(
        layout, G, M, N, K, _ptr(a), _ptr(a_scales), _q(Q_E4M3_1x128), _ptr(b), _ptr(b_scales), _q(b_qdesc),
        _ptr(offsets), _ptr(masked_m), _ptr(out), out.stride(-2), _stream(dev))
    _check("fgg_grouped_gemm_scaled", st)
    return out


def grouped_gemm_silu_quantize(a, a_scales, b, b_scales, offsets, counts=None, out=None, scales=None):
    """Gate-up grouped GEMM with SiLU(gate)*up and the 1x128 e4m3 requantization
    fused (fgg_grouped_gemm_silu_quantize): a [M, K] e4m3 with [K/128, M]
    scales, b [G, 2I, K] ([gate | up] rows) with [G, 2I/128, K/128] scales.
    ``counts`` (optional, [G] int32): real rows per group; padding rows past
    them are not written.  Returns (codes uint8 [M, I], scales f32 [I/128, M])."""
    G, N2, K = b.shape
    I = N2 // 2
    M = a.shape[0]
    dev = a.device
    for t in (a, a_scales, b, b_scales, offsets):
        assert t.is_contiguous()
    if out is None:
        out = torch.empty((M, I), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((I // 128, M), dtype=torch.float32, device=dev)
    st = load_library().fgg_grouped_gemm_silu_quantize(
        G, M, I, K, _ptr(a), _ptr(a_scales), _q(Q_E4M3_1x128), _ptr(b), _ptr(b_scales), _q(Q_E4M3_128x128),
        _ptr(offsets), _ptr(counts), _ptr(out), _ptr(scales), _stream(dev))
    _check("fgg_grouped_gemm_silu_quantize", st)
    return out, scales


def pack_fp4_weights(b, b_scales, out=None, scales_out=None):
    """Re-lay out FP4 expert weights for the masked GEMM (fgg_pack_fp4_weights):
    b [G, N, K/2] uint8 E2M1 pairs and b_scales [G, N, K/32] uint8 E8M0 ->
    (b_tiled uint8 [G, N*K/2], s_tiled uint8 [G, (N/16)*ceil(K/512)*256]), used with
    b_qdesc=Q_E2M1_E8M0_1x32_TILED."""
    G, N, Kh = b.shape
    K = 2 * Kh
    for t in (b, b_scales):
        assert t.is_contiguous()
    lib = load_library()
    nb, ns = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("fgg_pack_fp4_weights_bytes", lib.fgg_pack_fp4_weights_bytes(G, N, K, ctypes.byref(nb), ctypes.byref(ns)))
    dev = b.device
    if out is None:
        out = torch.empty((G, nb.value // max(G, 1)), dtype=torch.uint8, device=dev)
    if scales_out is None:
        scales_out = torch.empty((G, ns.value // max(G, 1)), dtype=torch.uint8, device=dev)
    assert out.numel() >= nb.value and scales_out.numel() >= ns.value
    st = lib.fgg_pack_fp4_weights(_ptr(b), _ptr(b_scales), G, N, K, _ptr(out), _ptr(scales_out), _stream(dev))
    _check("fgg_pack_fp4_weights", st)
    return out, scales_out


def _scaled_qdescs(qdesc):
    return {"fp8": (Q_E4M3_1x128, Q_E4M3_128x128), "w4a4": (Q_E2M1_1x16, Q_E2M1_1x16),
            "mxfp4": (Q_E2M1_E8M0_1x32, Q_E2M1_E8M0_1x32)}[qdesc]


def scaled_gemm_workspace_bytes(M: int, N: int, K: int, qdesc: str = "fp8", rank: int = 0) -> int:
    """Workspace bytes scaled_gemm needs (fgg_scaled_gemm_workspace)."""
    aq, bq = _scaled_qdescs(qdesc)
    epi = Epilogue(None, None, None, int(rank), None)
    n = ctypes.c_size_t(0)
    _check("fgg_scaled_gemm_workspace", load_library().fgg_scaled_gemm_workspace(
        M, N, K, _q(aq), _q(bq), ctypes.byref(epi), ctypes.byref(n)))
    return n.value


def scaled_gemm(a, a_scales, b, b_scales, qdesc="fp8", x_bf16=None, l_down=None, l_up=None, bias=None,
                out=None, workspace=None):
    """Dense case.  qdesc "fp8": a [M, K] e4m3 with [K/128, M] scales, b [N, K]
    with [N/128, K/128] scales.  qdesc "w4a4": a [M, K/2], b [N, K/2] packed
    E2M1 with [rows, K/16] fp32 scales; qdesc "mxfp4": the same codes with
    [rows, K/32] E8M0 scale bytes.  Both FP4 forms take an optional low-rank
    branch (x_bf16 [M, K], l_down [K, r], l_up [r, N], r = 32) and bias [N] (bf16)."""
    dev = a.device
    M = a.shape[0]
    N = b.shape[0]
    aq, bq = _scaled_qdescs(qdesc)
    K = a.shape[1] if qdesc == "fp8" else a.shape[1] * 2
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    epi = None
    if qdesc != "fp8" and (l_down is not None or bias is not None):
        rank = 0 if l_down is None else int(l_down.shape[1])
        epi = Epilogue(None if x_bf16 is None else x_bf16.data_ptr(),
                       None if l_down is None else l_down.data_ptr(),
                       None if l_up is None else l_up.data_ptr(), rank,
                       None if bias is None else bias.data_ptr())
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    _check("fgg_scaled_gemm_workspace", lib.fgg_scaled_gemm_workspace(
        M, N, K, _q(aq), _q(bq), ctypes.byref(epi) if epi is not None else None, ctypes.byref(nbytes)))
    if workspace is None and nbytes.value > 0:
        workspace = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    st = lib.fgg_scaled_gemm(M, N, K, _ptr(a), _ptr(a_scales), _q(aq), _ptr(b), _ptr(b_scales), _q(bq),
                             ctypes.byref(epi) if epi is not None else None, _ptr(out), out.stride(0),
                             _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev))
    _check("fgg_scaled_gemm", st)
    return out


def moe_combine(y, src_to_row, topk_w, out=None):
    """out[t] = Σ_j w[t, j] · y[src_to_row[t·k + j]] (bf16 [T, N])."""
    T, k = topk_w.shape
    N = y.shape[1]
    dev = y.device
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    st = load_library().fgg_moe_combine(_ptr(y), y.stride(0), _ptr(src_to_row), _ptr(topk_w), T, k, N,
                                         _ptr(out), out.stride(0), _stream(dev))
    _check("fgg_moe_combine", st)
    return out


def moe_down_combine_workspace_bytes(M: int) -> int:
    n = ctypes.c_size_t(0)
    _check("fgg_moe_down_combine_workspace", load_library().fgg_moe_down_combine_workspace(M, ctypes.byref(n)))
    return n.value


def moe_down_combine(a, a_scales, b, b_scales, offsets, counts, src_to_row, row_to_src, topk_w, y, out=None,
                     workspace=None):
    """Down GEMM and combine in one call (fgg_moe_down_combine): ``out`` equals
    ``moe_combine(grouped_gemm_scaled(a, ..., offsets, masked_m=counts), src_to_row, topk_w)``
    bit for bit.  ``y`` (bf16 [M, N]) receives the rows of tokens with two or more
    routed slots; rows of single-slot tokens go straight to ``out`` (bf16 [T, N])."""
    G, N, K = b.shape
    M = a.shape[0]
    T, k = topk_w.shape
    dev = a.device
    for t in (a, a_scales, b, b_scales, offsets, counts, src_to_row, row_to_src, topk_w):
        assert t.is_contiguous()
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_down_combine_workspace_bytes(M), dtype=torch.uint8, device=dev)
    st = load_library().fgg_moe_down_combine(
        G, M, N, K, _ptr(a), _ptr(a_scales), _q(Q_E4M3_1x128), _ptr(b), _ptr(b_scales), _q(Q_E4M3_128x128),
        _ptr(offsets), _ptr(counts), _ptr(src_to_row), _ptr(row_to_src), _ptr(topk_w), T, k, _ptr(y), y.stride(0),
        _ptr(workspace), workspace.numel(), _ptr(out), out.stride(0), _stream(dev))
    _check("fgg_moe_down_combine", st)
    return out
