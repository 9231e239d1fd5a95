// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
// Callers have validated every argument; these functions only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fgg {

// Static description of one kernel instance: its workgroup tile, threads and LDS
// budget.  [W4A4] §6 traces a silent slowdown to a shared-memory budget that was
// counted wrong (one buffer left out), and asks for every stage/buffer choice to be
// tabulated and checked; lds_bytes = stages * stage_bytes + other_bytes is the
// kernel's declared static LDS, which a test compares with the compiled kernel's.
struct KernelInfo {
  const char* name;      // kernel instance
  const char* entry;     // C entry point(s) that launch it
  int tile_m, tile_n, tile_k;   // workgroup tile (0: not a tiled kernel)
  int threads;           // threads per workgroup
  int stages;            // LDS ring stages (0: no ring)
  int stage_bytes;       // LDS bytes per stage
  int other_bytes;       // LDS outside the ring: group tables, scale caches, reductions
  int lds_bytes;         // declared static LDS
  const void* fn;        // the kernel (for hipFuncGetAttributes)
};

// Every kernel of the library, in a fixed order.
int kernel_table(const KernelInfo* const** out);

// FGG_DEBUG (environment, read once): one line per kernel launch on stderr with the
// kernel, the problem, grid, threads, tile, LDS bytes and stages.
bool debug_enabled();
void trace_launch(const KernelInfo& k, dim3 grid, const char* fmt, ...) __attribute__((format(printf, 3, 4)));

extern const KernelInfo kInfoQuantE4m3_1x128, kInfoQuantE4m3_128x128, kInfoQuantE2m1_1x16,
    kInfoQuantE2m1E8m0_1x32, kInfoPermuteHist, kInfoPermuteScan, kInfoPermuteScatter, kInfoPermuteGather,
    kInfoPermuteQuantize, kInfoFill, kInfoCombine, kInfoCombineRows, kInfoCombineRest, kInfoFp8Contig,
    kInfoFp8ContigSilu, kInfoFp8ContigCombine, kInfoFp8Dense,
    kInfoMaskedFp4Tiled, kInfoMaskedFp4, kInfoMaskedFp8, kInfoPackFp4, kInfoPackFp4Scales, kInfoW4a4Prep, kInfoW4a4LowRank,
    kInfoW4a4Gemm, kInfoMxfp4Gemm;

enum class QuantKind { E4M3_1x128, E4M3_128x128, E2M1_1x16, E2M1_E8M0_1x32 };

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ldx,
                           QuantKind kind, bool silu, const int32_t* rows_dev, void* q, void* scales,
                           int num_cus, hipStream_t st);

// Permute workspace layout (bytes): hist[nblk][E] int32, base[nblk][E] int32.
size_t permute_workspace_bytes(int64_t T, int32_t k, int32_t E);
hipError_t launch_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t align,
                          const uint8_t* xq, const float* xs, int64_t K, int32_t* offsets,
                          int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, uint8_t* a_out,
                          float* sa_out, int64_t M_cap, void* ws, hipStream_t st);

// The no-allocation permute's scratch: a file-scope device array of this many bytes
// (holds the permute workspace of up to (kPermuteScratchBytes - 256) / 4 histogram
// entries, ceil(T·k / 256) · E); permute_scratch gives its device address on the
// current device (taken once per device).
constexpr size_t kPermuteScratchBytes = size_t(2) << 20;
hipError_t permute_scratch(void** ptr);

hipError_t launch_permute_quantize(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                   const void* x, bool bf16, int64_t K, int64_t ldx, int32_t* offsets,
                                   int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, uint8_t* a_out,
                                   float* sa_out, int64_t M_cap, void* ws, int num_cus, hipStream_t st);
hipError_t launch_combine(const uint16_t* y, int64_t ldy, const int32_t* src_to_row, const float* w,
                          int64_t T, int32_t k, int64_t N, uint16_t* out, int64_t ldo,
                          hipStream_t st);
// The down GEMM with the combine of single-slot tokens in its epilogue: the routing
// table (row_info, roundup(M, 128) entries of 8 bytes: token or -1, weight), the GEMM,
// then the combine of the other tokens.
hipError_t launch_combine_rows(const int32_t* row_to_src, const int32_t* src_to_row, const float* w, int64_t T,
                               int32_t k, int64_t M, uint8_t* row_info, hipStream_t st);
hipError_t launch_gemm_fp8_combine(int32_t G, int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                                   const uint8_t* b, const float* sb, const int32_t* offsets, const int32_t* valid,
                                   uint16_t* y, int64_t ldy, const uint8_t* row_info, uint16_t* out, int64_t ldo,
                                   int num_cus, hipStream_t st);
hipError_t launch_combine_rest(const uint16_t* y, int64_t ldy, const int32_t* src_to_row, const float* w, int64_t T,
                               int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t st);

// FP8 x FP8 grouped GEMM, contiguous layout (dense = one group with offsets {0, M}).
// If offsets == nullptr the single group covers rows [0, M).  valid (nullable, with
// offsets only): per-group row counts; rows past offsets[g] + valid[g] are padding.
hipError_t launch_gemm_fp8_contig(int32_t G, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                  const float* sa, const uint8_t* b, const float* sb,
                                  const int32_t* offsets, const int32_t* valid, uint16_t* d, int64_t ldd,
                                  int num_cus, hipStream_t st);

// The gate-up grouped GEMM with the SiLU(gate)*up 1x128 e4m3 requantization epilogue.
hipError_t launch_gemm_fp8_silu_quantize(int32_t G, int64_t M, int64_t I, int64_t K, const uint8_t* a,
                                         const float* sa, const uint8_t* b, const float* sb,
                                         const int32_t* offsets, const int32_t* valid, uint8_t* q, float* s,
                                         int num_cus, hipStream_t st);

// Masked (decode) layout, A e4m3 1x128; B either E2M1x2 + E8M0/32 or e4m3 128x128.
hipError_t launch_gemm_masked(bool b_fp4, bool tiled, int32_t G, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, const float* sa, const uint8_t* b, const void* sb,
                              const int32_t* masked_m, uint16_t* d, int64_t ldd, hipStream_t st);

// FP4 weight tiling for the decode kernel: codes [G][N][K/2] and E8M0 scales [G][N][K/32]
// to FGG_E2M1X2_TILED codes and their scale spans (sizes from fp4_tiled_bytes).
void fp4_tiled_bytes(int32_t G, int64_t N, int64_t K, size_t* b_bytes, size_t* s_bytes);
hipError_t launch_pack_fp4(int32_t G, int64_t N, int64_t K, const uint8_t* b, const uint8_t* s, uint8_t* bt,
                           uint8_t* st, int num_cus, hipStream_t stream);

// W4A4: E2M1 x E2M1 with fp32 per-16 scales, optional rank-r low-rank branch and bias.
size_t w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank);
hipError_t launch_w4a4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, const uint16_t* x_bf16,
                       const uint16_t* l_down, const uint16_t* l_up, int32_t rank,
                       const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, int num_cus, hipStream_t st);

// T = bf16(X · L_down), rank 32 ([M][32]), by w4a4_lowrank_kernel (sixteen waves per 16 rows).
hipError_t launch_lowrank_t(int64_t M, int64_t K, const uint16_t* x_bf16, const uint16_t* l_down, uint16_t* T,
                            hipStream_t st);

// MXFP4 A4W4: E2M1 with E8M0 per 32 on both operands (scales [rows][K/32] bytes), optional
// rank-32 low-rank branch (workspace: T [M][32] bf16) and bias.
size_t mxfp4_workspace_bytes(int64_t M, int32_t rank);
hipError_t launch_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                        const uint8_t* sb, const uint16_t* x_bf16, const uint16_t* l_down, const uint16_t* l_up,
                        int32_t rank, const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, hipStream_t st);

}  // namespace fgg
