// C ABI of libfgg.so: argument validation, device check and dispatch to the
// kernels.  Every entry point either returns an error before launching
// anything or enqueues its kernels on the caller's stream and returns.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fgg.h"
#include "fgg_internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<int> g_num_cus_override{0};

constexpr int kMaxDevices = 64;
struct DeviceInfo {
  std::once_flag once;
  bool gfx950 = false;
  int num_cus = 0;
};
DeviceInfo g_dev[kMaxDevices];

fgg_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return FGG_ERR_HIP;
}

// Current device must be gfx950; fills num_cus.
fgg_status device_check(int* num_cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return FGG_ERR_UNSUPPORTED;
  DeviceInfo& d = g_dev[dev];
  std::call_once(d.once, [&] {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return;
    d.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = p.multiProcessorCount;
  });
  if (!d.gfx950) return FGG_ERR_UNSUPPORTED;
  const int ov = g_num_cus_override.load();
  if (num_cus) *num_cus = ov > 0 ? ov : d.num_cus;
  return FGG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool same_q(const fgg_qdesc& q, fgg_dtype data, fgg_dtype scale, int br, int bk) {
  return q.data == data && q.scale == scale && q.block_rows == br && q.block_k == bk;
}

fgg_status finish(hipError_t e) { return e == hipSuccess ? FGG_OK : hip_fail(e); }

}  // namespace

namespace fgg {

bool debug_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("FGG_DEBUG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

void trace_launch(const KernelInfo& k, dim3 grid, const char* fmt, ...) {
  if (!debug_enabled()) return;
  char what[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(what, sizeof what, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[fgg] %s: %s | grid=%u threads=%d tile=%dx%dx%d lds=%d B (%d x %d stage + %d) \n", k.name,
               what, grid.x * grid.y * grid.z, k.threads, k.tile_m, k.tile_n, k.tile_k, k.lds_bytes, k.stages,
               k.stage_bytes, k.other_bytes);
}

int kernel_table(const KernelInfo* const** out) {
  static const KernelInfo* const table[] = {
      &kInfoQuantE4m3_1x128, &kInfoQuantE4m3_128x128, &kInfoQuantE2m1_1x16, &kInfoQuantE2m1E8m0_1x32,
      &kInfoPermuteHist,     &kInfoPermuteScan,       &kInfoPermuteScatter, &kInfoPermuteGather,
      &kInfoPermuteQuantize, &kInfoFill,              &kInfoCombine,        &kInfoCombineRows,
      &kInfoCombineRest,     &kInfoFp8Contig,         &kInfoFp8ContigSilu,  &kInfoFp8ContigCombine,
      &kInfoFp8Dense,        &kInfoMaskedFp4Tiled,    &kInfoMaskedFp4,
      &kInfoMaskedFp8,       &kInfoPackFp4,           &kInfoPackFp4Scales,  &kInfoW4a4Prep,
      &kInfoW4a4LowRank,     &kInfoW4a4Gemm,         &kInfoMxfp4Gemm,
  };
  *out = table;
  return (int)(sizeof table / sizeof table[0]);
}

}  // namespace fgg

// The C ABI is the library's only export (the build hides everything else).
#pragma GCC visibility push(default)
extern "C" {

const char* fgg_status_string(fgg_status s) {
  switch (s) {
    case FGG_OK: return "FGG_OK";
    case FGG_ERR_INVALID_VALUE: return "FGG_ERR_INVALID_VALUE";
    case FGG_ERR_UNSUPPORTED: return "FGG_ERR_UNSUPPORTED";
    case FGG_ERR_HIP: return "FGG_ERR_HIP";
  }
  return "FGG_ERR_UNKNOWN";
}

int fgg_last_hip_error(void) { return g_last_hip_error; }

fgg_status fgg_set_num_cus(int n) {
  if (n < 0) return FGG_ERR_INVALID_VALUE;
  g_num_cus_override.store(n);
  return FGG_OK;
}

fgg_status fgg_quantize_blockwise(const void* x, fgg_dtype x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  fgg_act act, fgg_qdesc q, const int32_t* rows_dev, void* q_out, void* scales_out,
                                  void* stream) {
  if (rows < 0 || cols < 0) return FGG_ERR_INVALID_VALUE;
  if (x_dtype != FGG_F32 && x_dtype != FGG_BF16) return FGG_ERR_UNSUPPORTED;
  if (act != FGG_ACT_NONE && act != FGG_ACT_SILU_MUL) return FGG_ERR_INVALID_VALUE;
  fgg::QuantKind kind;
  if (same_q(q, FGG_E4M3, FGG_F32, 1, 128)) kind = fgg::QuantKind::E4M3_1x128;
  else if (same_q(q, FGG_E4M3, FGG_F32, 128, 128)) kind = fgg::QuantKind::E4M3_128x128;
  else if (same_q(q, FGG_E2M1X2, FGG_F32, 1, 16)) kind = fgg::QuantKind::E2M1_1x16;
  else if (same_q(q, FGG_E2M1X2, FGG_E8M0, 1, 32)) kind = fgg::QuantKind::E2M1_E8M0_1x32;
  else return FGG_ERR_UNSUPPORTED;
  const bool silu = act == FGG_ACT_SILU_MUL;
  if (silu && kind != fgg::QuantKind::E4M3_1x128) return FGG_ERR_UNSUPPORTED;
  if (rows_dev && kind != fgg::QuantKind::E4M3_1x128) return FGG_ERR_UNSUPPORTED;
  if (cols % q.block_k != 0) return FGG_ERR_UNSUPPORTED;
  if (q.block_rows == 128 && rows % 128 != 0) return FGG_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return FGG_OK;
  if (!x || !q_out || !scales_out) return FGG_ERR_INVALID_VALUE;
  const int64_t need = silu ? 2 * cols : cols;
  if (ldx < need) return FGG_ERR_INVALID_VALUE;
  const int64_t esz = x_dtype == FGG_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esz) % 16 != 0 || !aligned(q_out, 16) || !aligned(scales_out, 4))
    return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  fgg_status st = device_check(&num_cus);
  if (st != FGG_OK) return st;
  return finish(fgg::launch_quantize(x, x_dtype == FGG_BF16, rows, cols, ldx, kind, silu, rows_dev, q_out,
                                     scales_out, num_cus, (hipStream_t)stream));
}

fgg_status fgg_moe_permute_workspace(int64_t T, int32_t k, int32_t E, size_t* bytes) {
  if (!bytes || T < 0 || k < 1 || k > 64 || E < 1 || E > 1024) return FGG_ERR_INVALID_VALUE;
  *bytes = fgg::permute_workspace_bytes(T, k, E);
  return FGG_OK;
}

fgg_status fgg_moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                           const void* xq, const float* xs, int64_t K, int32_t* offsets, int32_t* counts,
                           int32_t* src_to_row, int32_t* row_to_src, void* a_out, float* sa_out,
                           int64_t M_cap, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > 1024 || align < 1 || align > 1024 || M_cap < 0)
    return FGG_ERR_INVALID_VALUE;
  if (!offsets || !counts) return FGG_ERR_INVALID_VALUE;
  if (T > 0 && (!topk_ids || !src_to_row)) return FGG_ERR_INVALID_VALUE;
  if (M_cap > 0 && !row_to_src) return FGG_ERR_INVALID_VALUE;
  if (T * (int64_t)k > (int64_t)INT32_MAX || M_cap > (int64_t)INT32_MAX) return FGG_ERR_UNSUPPORTED;
  if (xq) {
    if (K <= 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
    if (!xs || !a_out || !sa_out) return FGG_ERR_INVALID_VALUE;
    if (!aligned(xq, 16) || !aligned(a_out, 16) || !aligned(xs, 4) || !aligned(sa_out, 4))
      return FGG_ERR_INVALID_VALUE;
  }
  if (T > 0 && (!workspace || ws_bytes < fgg::permute_workspace_bytes(T, k, E))) return FGG_ERR_INVALID_VALUE;
  fgg_status st = device_check(nullptr);
  if (st != FGG_OK) return st;
  return finish(fgg::launch_permute(topk_ids, T, k, E, align, (const uint8_t*)xq, xs, K, offsets, counts,
                                    src_to_row, row_to_src, (uint8_t*)a_out, sa_out, M_cap, workspace,
                                    (hipStream_t)stream));
}

fgg_status fgg_moe_permute_quantize(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                    const void* x, fgg_dtype x_dtype, int64_t K, int64_t ldx, int32_t* offsets,
                                    int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, void* a_out,
                                    float* sa_out, int64_t M_cap, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > 1024 || align < 1 || align > 1024 || M_cap < 0 || K < 0)
    return FGG_ERR_INVALID_VALUE;
  if (x_dtype != FGG_BF16 && x_dtype != FGG_F32) return FGG_ERR_UNSUPPORTED;
  if (K == 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
  if (!offsets || !counts) return FGG_ERR_INVALID_VALUE;
  if (T > 0 && (!topk_ids || !src_to_row || !x)) return FGG_ERR_INVALID_VALUE;
  if (M_cap > 0 && (!row_to_src || !a_out || !sa_out)) return FGG_ERR_INVALID_VALUE;
  if (T * (int64_t)k > (int64_t)INT32_MAX || M_cap > (int64_t)INT32_MAX) return FGG_ERR_UNSUPPORTED;
  const int64_t esz = x_dtype == FGG_F32 ? 4 : 2;
  if (T > 0 && (ldx < K || !aligned(x, 16) || (ldx * esz) % 16 != 0)) return FGG_ERR_INVALID_VALUE;
  if (M_cap > 0 && (!aligned(a_out, 16) || !aligned(sa_out, 4))) return FGG_ERR_INVALID_VALUE;
  if (T > 0 && (!workspace || ws_bytes < fgg::permute_workspace_bytes(T, k, E))) return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  fgg_status st = device_check(&num_cus);
  if (st != FGG_OK) return st;
  return finish(fgg::launch_permute_quantize(topk_ids, T, k, E, align, x, x_dtype == FGG_BF16, K, ldx, offsets,
                                             counts, src_to_row, row_to_src, (uint8_t*)a_out, sa_out, M_cap,
                                             workspace, num_cus, (hipStream_t)stream));
}

fgg_status fgg_moe_permute_quantize_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                            const void* x, fgg_dtype x_dtype, int64_t K, int64_t ldx,
                                            int32_t* offsets, int32_t* counts, int32_t* src_to_row,
                                            int32_t* row_to_src, void* a_out, float* sa_out, int64_t M_cap,
                                            void* stream) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > 1024) return FGG_ERR_INVALID_VALUE;
  if (T > 0 && fgg::permute_workspace_bytes(T, k, E) > fgg::kPermuteScratchBytes) return FGG_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (T > 0) {
    fgg_status st = device_check(nullptr);
    if (st != FGG_OK) return st;
    const hipError_t e = fgg::permute_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e);
  }
  return fgg_moe_permute_quantize(topk_ids, T, k, E, align, x, x_dtype, K, ldx, offsets, counts, src_to_row,
                                  row_to_src, a_out, sa_out, M_cap, ws, fgg::kPermuteScratchBytes, stream);
}

fgg_status fgg_grouped_gemm_scaled(fgg_layout layout, int32_t G, int64_t M, int64_t N, int64_t K,
                                   const void* a, const void* a_scales, fgg_qdesc aq, const void* b,
                                   const void* b_scales, fgg_qdesc bq, const int32_t* offsets,
                                   const int32_t* masked_m, void* d, int64_t ldd, void* stream) {
  if (G < 1 || G > 1024 || M < 0 || N < 0 || K < 0) return FGG_ERR_INVALID_VALUE;
  if (N % 128 != 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
  if (ldd < N || ldd % 8 != 0) return FGG_ERR_INVALID_VALUE;
  if (!same_q(aq, FGG_E4M3, FGG_F32, 1, 128)) return FGG_ERR_UNSUPPORTED;
  // (with K == 0 the operands hold no bytes and are never read: they may be NULL)
  if ((K > 0 && (!a || !a_scales || !b || !b_scales)) || !d) return FGG_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4))
    return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  if (layout == FGG_LAYOUT_CONTIGUOUS) {
    if (!same_q(bq, FGG_E4M3, FGG_F32, 128, 128)) return FGG_ERR_UNSUPPORTED;
    if (K > 16384) return FGG_ERR_UNSUPPORTED;
    if (!offsets) return FGG_ERR_INVALID_VALUE;
    fgg_status st = device_check(&num_cus);
    if (st != FGG_OK) return st;
    if (M == 0 || N == 0) return FGG_OK;
    return finish(fgg::launch_gemm_fp8_contig(G, M, N, K, (const uint8_t*)a, (const float*)a_scales,
                                              (const uint8_t*)b, (const float*)b_scales, offsets, masked_m,
                                              (uint16_t*)d, ldd, num_cus, (hipStream_t)stream));
  }
  if (layout == FGG_LAYOUT_MASKED) {
    const bool tiled = same_q(bq, FGG_E2M1X2_TILED, FGG_E8M0, 1, 32);
    const bool fp4 = tiled || same_q(bq, FGG_E2M1X2, FGG_E8M0, 1, 32);
    if (!fp4 && !same_q(bq, FGG_E4M3, FGG_F32, 128, 128)) return FGG_ERR_UNSUPPORTED;
    if (M > 16 || K == 0) return FGG_ERR_UNSUPPORTED;
    if (!masked_m) return FGG_ERR_INVALID_VALUE;
    if (tiled && !aligned(b_scales, 16)) return FGG_ERR_INVALID_VALUE;
    fgg_status st = device_check(&num_cus);
    if (st != FGG_OK) return st;
    if (M == 0 || N == 0) return FGG_OK;
    return finish(fgg::launch_gemm_masked(fp4, tiled, G, M, N, K, (const uint8_t*)a, (const float*)a_scales,
                                          (const uint8_t*)b, b_scales, masked_m, (uint16_t*)d, ldd,
                                          (hipStream_t)stream));
  }
  return FGG_ERR_INVALID_VALUE;
}

fgg_status fgg_grouped_gemm_silu_quantize(int32_t G, int64_t M, int64_t I, int64_t K, const void* a,
                                          const void* a_scales, fgg_qdesc aq, const void* b, const void* b_scales,
                                          fgg_qdesc bq, const int32_t* offsets, const int32_t* counts, void* q_out,
                                          float* s_out, void* stream) {
  if (G < 1 || G > 1024 || M < 0 || I < 0 || K < 0) return FGG_ERR_INVALID_VALUE;
  if (I % 128 != 0 || K % 128 != 0 || K > 16384) return FGG_ERR_UNSUPPORTED;
  if (!same_q(aq, FGG_E4M3, FGG_F32, 1, 128) || !same_q(bq, FGG_E4M3, FGG_F32, 128, 128)) return FGG_ERR_UNSUPPORTED;
  if ((K > 0 && (!a || !a_scales || !b || !b_scales)) || !offsets || !q_out || !s_out) return FGG_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(q_out, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(s_out, 4))
    return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  fgg_status st = device_check(&num_cus);
  if (st != FGG_OK) return st;
  if (M == 0 || I == 0) return FGG_OK;
  return finish(fgg::launch_gemm_fp8_silu_quantize(G, M, I, K, (const uint8_t*)a, (const float*)a_scales,
                                                   (const uint8_t*)b, (const float*)b_scales, offsets, counts,
                                                   (uint8_t*)q_out, s_out, num_cus, (hipStream_t)stream));
}

fgg_status fgg_scaled_gemm_workspace(int64_t M, int64_t N, int64_t K, fgg_qdesc aq, fgg_qdesc bq,
                                     const fgg_epilogue* epi, size_t* bytes) {
  if (!bytes || M < 0 || N < 0 || K < 0) return FGG_ERR_INVALID_VALUE;
  *bytes = 0;
  if (same_q(aq, FGG_E2M1X2, FGG_F32, 1, 16) && same_q(bq, FGG_E2M1X2, FGG_F32, 1, 16))
    *bytes = fgg::w4a4_workspace_bytes(M, N, K, epi ? epi->rank : 0);
  if (same_q(aq, FGG_E2M1X2, FGG_E8M0, 1, 32) && same_q(bq, FGG_E2M1X2, FGG_E8M0, 1, 32))
    *bytes = fgg::mxfp4_workspace_bytes(M, epi ? epi->rank : 0);
  return FGG_OK;
}

fgg_status fgg_scaled_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* a_scales, fgg_qdesc aq,
                           const void* b, const void* b_scales, fgg_qdesc bq, const fgg_epilogue* epi, void* d,
                           int64_t ldd, void* workspace, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FGG_ERR_INVALID_VALUE;
  // (N % 128 for the FP8 and per-16 W4A4 paths, N % 16 for MXFP4: checked per path below)
  if (N % 16 != 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
  if (ldd < N || ldd % 8 != 0) return FGG_ERR_INVALID_VALUE;
  // (with K == 0 the operands hold no bytes and are never read: they may be NULL)
  if ((K > 0 && (!a || !a_scales || !b || !b_scales)) || !d) return FGG_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4))
    return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  if (same_q(aq, FGG_E4M3, FGG_F32, 1, 128) && same_q(bq, FGG_E4M3, FGG_F32, 128, 128)) {
    if (epi || N % 128 != 0) return FGG_ERR_UNSUPPORTED;
    if (K > 16384) return FGG_ERR_UNSUPPORTED;
    fgg_status st = device_check(&num_cus);
    if (st != FGG_OK) return st;
    if (M == 0 || N == 0) return FGG_OK;
    return finish(fgg::launch_gemm_fp8_contig(1, M, N, K, (const uint8_t*)a, (const float*)a_scales,
                                              (const uint8_t*)b, (const float*)b_scales, nullptr, nullptr,
                                              (uint16_t*)d, ldd, num_cus, (hipStream_t)stream));
  }
  if (same_q(aq, FGG_E2M1X2, FGG_F32, 1, 16) && same_q(bq, FGG_E2M1X2, FGG_F32, 1, 16)) {
    // (the GEMM's per-lane DMA offsets are 32-bit: 128 rows x 2K bytes)
    if (M % 128 != 0 || N % 128 != 0 || K == 0 || K > (int64_t(1) << 22)) return FGG_ERR_UNSUPPORTED;
    if (!aligned(a_scales, 8) || !aligned(b_scales, 8)) return FGG_ERR_INVALID_VALUE;
    const int32_t rank = epi ? epi->rank : 0;
    if (rank != 0 && rank != 32) return FGG_ERR_UNSUPPORTED;
    if (rank == 32) {
      if (!epi->x_bf16 || !epi->l_down || !epi->l_up) return FGG_ERR_INVALID_VALUE;
      if (!aligned(epi->x_bf16, 16) || !aligned(epi->l_down, 2) || !aligned(epi->l_up, 2))
        return FGG_ERR_INVALID_VALUE;
    }
    if (M > 0 && N > 0 &&
        (!workspace || ws_bytes < fgg::w4a4_workspace_bytes(M, N, K, rank) || !aligned(workspace, 256)))
      return FGG_ERR_INVALID_VALUE;
    const void* bias = epi ? epi->bias : nullptr;
    if (bias && !aligned(bias, 2)) return FGG_ERR_INVALID_VALUE;
    fgg_status st = device_check(&num_cus);
    if (st != FGG_OK) return st;
    if (M == 0 || N == 0) return FGG_OK;
    return finish(fgg::launch_w4a4(M, N, K, (const uint8_t*)a, (const float*)a_scales, (const uint8_t*)b,
                                   (const float*)b_scales, rank ? (const uint16_t*)epi->x_bf16 : nullptr,
                                   rank ? (const uint16_t*)epi->l_down : nullptr,
                                   rank ? (const uint16_t*)epi->l_up : nullptr, rank, (const uint16_t*)bias,
                                   (uint16_t*)d, ldd, workspace, num_cus, (hipStream_t)stream));
  }
  if (same_q(aq, FGG_E2M1X2, FGG_E8M0, 1, 32) && same_q(bq, FGG_E2M1X2, FGG_E8M0, 1, 32)) {
    // (per-lane DMA offsets are 32-bit: 256 rows x K/2 bytes)
    if (K == 0 || K > (int64_t(1) << 24)) return FGG_ERR_UNSUPPORTED;
    // (scale rows are read as dwords: K/32 bytes per row, a multiple of 4)
    const int32_t rank = epi ? epi->rank : 0;
    if (rank != 0 && rank != 32) return FGG_ERR_UNSUPPORTED;
    if (rank == 32) {
      if (!epi->x_bf16 || !epi->l_down || !epi->l_up) return FGG_ERR_INVALID_VALUE;
      if (!aligned(epi->x_bf16, 16) || !aligned(epi->l_down, 2) || !aligned(epi->l_up, 2))
        return FGG_ERR_INVALID_VALUE;
      if (M > 0 && N > 0 && (!workspace || ws_bytes < fgg::mxfp4_workspace_bytes(M, rank) || !aligned(workspace, 16)))
        return FGG_ERR_INVALID_VALUE;
    }
    const void* bias = epi ? epi->bias : nullptr;
    if (bias && !aligned(bias, 2)) return FGG_ERR_INVALID_VALUE;
    fgg_status st = device_check(&num_cus);
    if (st != FGG_OK) return st;
    if (M == 0 || N == 0) return FGG_OK;
    return finish(fgg::launch_mxfp4(M, N, K, (const uint8_t*)a, (const uint8_t*)a_scales, (const uint8_t*)b,
                                    (const uint8_t*)b_scales, rank ? (const uint16_t*)epi->x_bf16 : nullptr,
                                    rank ? (const uint16_t*)epi->l_down : nullptr,
                                    rank ? (const uint16_t*)epi->l_up : nullptr, rank, (const uint16_t*)bias,
                                    (uint16_t*)d, ldd, workspace, (hipStream_t)stream));
  }
  return FGG_ERR_UNSUPPORTED;
}

fgg_status fgg_pack_fp4_weights_bytes(int32_t G, int64_t N, int64_t K, size_t* b_bytes, size_t* s_bytes) {
  if (G < 0 || N < 0 || K < 0 || !b_bytes || !s_bytes) return FGG_ERR_INVALID_VALUE;
  if (N % 16 != 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
  fgg::fp4_tiled_bytes(G, N, K, b_bytes, s_bytes);
  return FGG_OK;
}

fgg_status fgg_pack_fp4_weights(const void* b, const void* b_scales, int32_t G, int64_t N, int64_t K,
                                void* b_tiled, void* s_tiled, void* stream) {
  if (G < 0 || N < 0 || K < 0) return FGG_ERR_INVALID_VALUE;
  if (N % 16 != 0 || K % 128 != 0) return FGG_ERR_UNSUPPORTED;
  const bool empty = G == 0 || N == 0 || K == 0;
  if (!empty && (!b || !b_scales || !b_tiled || !s_tiled)) return FGG_ERR_INVALID_VALUE;
  if (!aligned(b, 16) || !aligned(b_tiled, 16) || !aligned(s_tiled, 16)) return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  fgg_status st = device_check(&num_cus);
  if (st != FGG_OK) return st;
  if (empty) return FGG_OK;
  return finish(fgg::launch_pack_fp4(G, N, K, (const uint8_t*)b, (const uint8_t*)b_scales, (uint8_t*)b_tiled,
                                     (uint8_t*)s_tiled, num_cus, (hipStream_t)stream));
}

fgg_status fgg_moe_combine(const void* y, int64_t ldy, const int32_t* src_to_row, const float* topk_w, int64_t T,
                           int32_t k, int64_t N, void* out, int64_t ldo, void* stream) {
  if (T < 0 || k < 1 || k > 64 || N < 0) return FGG_ERR_INVALID_VALUE;
  if (N % 8 != 0) return FGG_ERR_UNSUPPORTED;
  if (ldy < N || ldo < N || ldy % 8 != 0 || ldo % 8 != 0) return FGG_ERR_INVALID_VALUE;
  if (T == 0 || N == 0) return FGG_OK;
  if (!y || !src_to_row || !topk_w || !out) return FGG_ERR_INVALID_VALUE;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_w, 4)) return FGG_ERR_INVALID_VALUE;
  fgg_status st = device_check(nullptr);
  if (st != FGG_OK) return st;
  return finish(fgg::launch_combine((const uint16_t*)y, ldy, src_to_row, topk_w, T, k, N, (uint16_t*)out, ldo,
                                    (hipStream_t)stream));
}

fgg_status fgg_moe_down_combine_workspace(int64_t M, size_t* bytes) {
  if (!bytes || M < 0) return FGG_ERR_INVALID_VALUE;
  *bytes = (size_t)((M + 127) / 128 * 128) * 8;
  return FGG_OK;
}

fgg_status fgg_moe_down_combine(int32_t G, int64_t M, int64_t N, int64_t K, const void* a, const void* a_scales,
                                fgg_qdesc aq, const void* b, const void* b_scales, fgg_qdesc bq,
                                const int32_t* offsets, const int32_t* counts, const int32_t* src_to_row,
                                const int32_t* row_to_src, const float* topk_w, int64_t T, int32_t k, void* y,
                                int64_t ldy, void* workspace, size_t ws_bytes, void* out, int64_t ldo,
                                void* stream) {
  if (G < 1 || G > 1024 || M < 0 || N < 0 || K < 0 || T < 0 || k < 1 || k > 64) return FGG_ERR_INVALID_VALUE;
  if (N % 128 != 0 || K % 128 != 0 || K > 16384) return FGG_ERR_UNSUPPORTED;
  if (!same_q(aq, FGG_E4M3, FGG_F32, 1, 128) || !same_q(bq, FGG_E4M3, FGG_F32, 128, 128)) return FGG_ERR_UNSUPPORTED;
  if (ldy < N || ldy % 8 != 0 || ldo < N || ldo % 8 != 0) return FGG_ERR_INVALID_VALUE;
  if ((K > 0 && (!a || !a_scales || !b || !b_scales)) || !offsets || !counts || !src_to_row || !row_to_src ||
      !topk_w || !y || !out)
    return FGG_ERR_INVALID_VALUE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(y, 16) || !aligned(out, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(topk_w, 4))
    return FGG_ERR_INVALID_VALUE;
  size_t need = 0;
  fgg_moe_down_combine_workspace(M, &need);
  if (M > 0 && (!workspace || !aligned(workspace, 16) || ws_bytes < need)) return FGG_ERR_INVALID_VALUE;
  int num_cus = 0;
  fgg_status st = device_check(&num_cus);
  if (st != FGG_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  uint8_t* ri = (uint8_t*)workspace;
  hipError_t e = fgg::launch_combine_rows(row_to_src, src_to_row, topk_w, T, k, M, ri, hs);
  if (e == hipSuccess)
    e = fgg::launch_gemm_fp8_combine(G, M, N, K, (const uint8_t*)a, (const float*)a_scales, (const uint8_t*)b,
                                     (const float*)b_scales, offsets, counts, (uint16_t*)y, ldy, ri, (uint16_t*)out,
                                     ldo, num_cus, hs);
  if (e == hipSuccess)
    e = fgg::launch_combine_rest((const uint16_t*)y, ldy, src_to_row, topk_w, T, k, N, (uint16_t*)out, ldo, hs);
  return finish(e);
}

int32_t fgg_kernel_count(void) {
  const fgg::KernelInfo* const* t = nullptr;
  return (int32_t)fgg::kernel_table(&t);
}

fgg_status fgg_kernel_info_get(int32_t i, fgg_kernel_info* info) {
  const fgg::KernelInfo* const* t = nullptr;
  const int n = fgg::kernel_table(&t);
  if (i < 0 || i >= n || !info) return FGG_ERR_INVALID_VALUE;
  const fgg::KernelInfo& k = *t[i];
  info->kernel = k.name;
  info->entry = k.entry;
  info->tile_m = k.tile_m;
  info->tile_n = k.tile_n;
  info->tile_k = k.tile_k;
  info->threads = k.threads;
  info->stages = k.stages;
  info->stage_bytes = k.stage_bytes;
  info->other_bytes = k.other_bytes;
  info->lds_bytes = k.lds_bytes;
  return FGG_OK;
}

fgg_status fgg_kernel_compiled_lds(int32_t i, int64_t* bytes) {
  const fgg::KernelInfo* const* t = nullptr;
  const int n = fgg::kernel_table(&t);
  if (i < 0 || i >= n || !bytes) return FGG_ERR_INVALID_VALUE;
  fgg_status st = device_check(nullptr);
  if (st != FGG_OK) return st;
  hipFuncAttributes attr;
  const hipError_t e = hipFuncGetAttributes(&attr, t[i]->fn);
  if (e != hipSuccess) return hip_fail(e);
  *bytes = (int64_t)attr.sharedSizeBytes;
  return FGG_OK;
}

}  // extern "C"
#pragma GCC visibility pop
