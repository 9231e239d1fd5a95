/*
 * fgg.h — block-scaled FP8/FP4 MoE grouped GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfgg.so.  Every pointer argument is a DEVICE pointer owned by the
 * caller unless stated otherwise; the library allocates nothing.  Every call
 * validates its arguments on the host, enqueues its kernels on `stream` (a
 * hipStream_t; NULL = the null stream) and returns without synchronizing.
 * Validation failures return a status without launching anything.
 *
 * Sources (web pages), cited by tag and section:
 *  [FP4MoE]   "Blackwell架构下FP4 MoE模型的TFLOPS性能优化" (intelliparadigm.com)
 *  [W4A4]     "最新GPU架构上W4A4算子的Warp专用化内核实践" (service.ruibaoantu.com)
 *  [Infra]    "腾讯 AI Infra" interview notes (ningzhengsheng.cn)
 *  [MegaMoE]  Hopper + DeepGEMM MoE article (www.mqxn.cn/news/59821)
 *  [DeepGEMM] DeepGEMM FP8 GEMM teardown (bhfrc.com/news/60438)
 *
 * Formats.  E4M3 is OCP FP8 e4m3 "FN" (max 448, 0x7F/0xFF NaN) — [DeepGEMM]
 * §2.1.  E2M1 is FP4 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) — [Infra] Q
 * "FP4量化是什么"; FGG_E2M1X2 packs two per byte, element 2i in the low nibble.
 * E8M0 is a power of two 2^(b-127).
 *
 * Scale layouts (fixed per quantization kind; chosen so that the GEMM kernels
 * read one contiguous run of scales per K block):
 *   E4M3, F32 scale, 1 × 128   (activations):  scales[K/128][rows]   (K-block-major)
 *   E4M3, F32 scale, 128 × 128 (weights):      scales[rows/128][K/128]
 *   E2M1X2, F32 scale, 1 × 16:                 scales[rows][K/16]
 *   E2M1X2, E8M0 scale, 1 × 32:                scales[rows][K/32] (uint8)
 * Code arrays are dense row-major: [rows][K] bytes (E4M3) or [rows][K/2] (E2M1X2).
 *
 * Thread safety: calls are stateless apart from fgg_set_num_cus(); calls on
 * different streams may run concurrently.  Errors from the HIP runtime are
 * reported as FGG_ERR_HIP; fgg_last_hip_error() then gives the hipError_t
 * (per host thread).
 */
#ifndef FGG_H_
#define FGG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FGG_OK = 0,
  FGG_ERR_INVALID_VALUE = 1, /* null required pointer, negative size, misaligned pointer, bad ld */
  FGG_ERR_UNSUPPORTED = 2,   /* valid but not implemented: shape not a multiple of the block, dtype combo, non-gfx950 device */
  FGG_ERR_HIP = 3            /* a HIP runtime call or kernel launch failed */
} fgg_status;

typedef enum {
  FGG_F32 = 0,
  FGG_BF16 = 1,
  FGG_E4M3 = 2,
  FGG_E2M1X2 = 3,
  FGG_E8M0 = 4,
  /* E2M1 codes packed as FGG_E2M1X2, stored in 16-row x 128-K tiles in MFMA operand
   * order (weights of the masked FP4 GEMM only; see fgg_pack_fp4_weights) */
  FGG_E2M1X2_TILED = 5
} fgg_dtype;

/* Quantization descriptor: code type, scale type and the block one scale covers. */
typedef struct {
  fgg_dtype data;     /* FGG_E4M3 or FGG_E2M1X2 */
  fgg_dtype scale;    /* FGG_F32 or FGG_E8M0 */
  int32_t block_rows; /* 1 or 128 */
  int32_t block_k;    /* 16, 32 or 128 */
} fgg_qdesc;

typedef enum { FGG_ACT_NONE = 0, FGG_ACT_SILU_MUL = 1 } fgg_act;
typedef enum { FGG_LAYOUT_CONTIGUOUS = 0, FGG_LAYOUT_MASKED = 1 } fgg_layout;

/* W4A4 epilogue ([W4A4] §1: Y = (Q(X)·Q(W)ᵀ) ⊙ scale + L(X) + b).  All fields may be NULL/0. */
typedef struct {
  const void* x_bf16; /* [M][K] bf16, row-major: the unquantized input read by the low-rank branch */
  const void* l_down; /* [K][rank] bf16, row-major */
  const void* l_up;   /* [rank][N] bf16, row-major */
  int32_t rank;       /* 0 (no low-rank branch) or 32 */
  const void* bias;   /* [N] bf16, the per-column affine term */
} fgg_epilogue;

/* Human-readable name of a status code (static string, never NULL). */
const char* fgg_status_string(fgg_status s);

/* hipError_t behind the last FGG_ERR_HIP returned on this host thread (0 if none). */
int fgg_last_hip_error(void);

/* Number of workgroup slots per "wave" of the persistent GEMM grids: the
 * compute-unit count the persistent kernels size their grid for
 * ([MegaMoE] §4.1 exposes the same knob as an SM count).  0 restores the
 * device's CU count.  Negative values: FGG_ERR_INVALID_VALUE. */
fgg_status fgg_set_num_cus(int n);

/*
 * Kernel table and launch trace ([MegaMoE] §4.2 prints each generated kernel's
 * configuration under a debug environment flag; [W4A4] §6 traces a throughput
 * loss to a shared-memory budget that left one buffer out, and asks for every
 * stage and buffer choice to be tabulated and checked).
 *
 * With the environment variable FGG_DEBUG set (not "0") when the library first
 * launches, every kernel launch prints one line on stderr: the kernel, the
 * problem (shape, dtype, options), grid, threads, workgroup tile and LDS budget.
 *
 * fgg_kernel_count / fgg_kernel_info_get describe every kernel of the library:
 * lds_bytes = stages * stage_bytes + other_bytes is the static LDS the kernel
 * declares (at most 160 KiB, the LDS of one gfx950 compute unit).  The strings
 * are static and owned by the library.  fgg_kernel_compiled_lds asks the HIP
 * runtime for the compiled kernel's static LDS (needs a gfx950 device; else
 * FGG_ERR_UNSUPPORTED).  An index outside [0, fgg_kernel_count()) or a NULL
 * output is FGG_ERR_INVALID_VALUE.
 */
typedef struct {
  const char* kernel;    /* kernel instance */
  const char* entry;     /* the entry point(s) that launch it */
  int32_t tile_m, tile_n, tile_k; /* workgroup tile (0 where the kernel is not tiled) */
  int32_t threads;       /* threads per workgroup */
  int32_t stages;        /* LDS ring stages (0: no ring) */
  int32_t stage_bytes;   /* LDS bytes per ring stage */
  int32_t other_bytes;   /* LDS outside the ring: group tables, scale caches, reductions */
  int32_t lds_bytes;     /* declared static LDS */
} fgg_kernel_info;

int32_t fgg_kernel_count(void);
fgg_status fgg_kernel_info_get(int32_t i, fgg_kernel_info* info);
fgg_status fgg_kernel_compiled_lds(int32_t i, int64_t* bytes);

/*
 * fgg_quantize_blockwise — online/offline block quantization.
 *
 * [Infra] Q "量化矩阵乘的维度和流程": every block shares one scale and the code
 * is round(x / scale); [DeepGEMM] §5.2: scale = max|x| / 448 for e4m3 (6 for
 * E2M1, its largest magnitude).  For each block:
 *   E4M3 / F32:  s = fl32(amax / 448); code = e4m3_rne_satfinite(fl32(x / s))
 *   E2M1 / F32:  s = fl32(amax / 6);   code = e2m1_rne_satfinite(fl32(x / s))
 *   E2M1 / E8M0: e = smallest integer with 6·2^e >= amax (clamped to
 *                [-127,127]); code = e2m1_rne(x · 2^-e); scale byte = e + 127
 * An all-zero block gets scale 1 (E8M0 byte 127).  Ties round to the even
 * code; magnitudes beyond the format's max saturate; signs (also of zero) are
 * kept.  Divisions are IEEE fp32.
 *
 * x:       [rows][ldx] elements of x_dtype (FGG_F32 or FGG_BF16); only the first
 *          `cols` (or 2·cols for FGG_ACT_SILU_MUL) of each row are read.
 * act:     FGG_ACT_SILU_MUL quantizes a = g / (1 + e^-g) · u computed in fp32,
 *          where row r holds [g | u] = x[r][0:cols], x[r][cols:2·cols]
 *          (SiLU of [MegaMoE] §3.1 on the gate half of a gate-up output);
 *          only with q = {E4M3, F32, 1, 128}.
 * q:       one of {E4M3,F32,1,128}, {E4M3,F32,128,128}, {E2M1X2,F32,1,16},
 *          {E2M1X2,E8M0,1,32}.
 * q_out:   codes, dense [rows][cols] (E4M3) or [rows][cols/2] (E2M1X2).
 * scales_out: in the layout of the quantization kind (see top of file).
 * rows_dev: optional DEVICE pointer to an int32 row count (e.g. offsets[E] of
 *          moe_permute); when non-NULL only rows < min(rows, *rows_dev) are
 *          read and written, so a caller can size `rows` for the worst case
 *          without a host synchronization.  Only with q = {E4M3, F32, 1, 128}.
 * Requires cols % block_k == 0 and, for 128-row blocks, rows % 128 == 0
 * (else FGG_ERR_UNSUPPORTED).  rows == 0 is a no-op.
 */
fgg_status fgg_quantize_blockwise(const void* x, fgg_dtype x_dtype, int64_t rows, int64_t cols,
                                  int64_t ldx, fgg_act act, fgg_qdesc q, const int32_t* rows_dev,
                                  void* q_out, void* scales_out, void* stream);

/*
 * fgg_moe_permute — expert histogram, padded prefix sum and stable scatter.
 *
 * [DeepGEMM] §5.3 (pass group ids and token offsets; keep each expert's rows
 * contiguous) and [FP4MoE] §4.2 (expert group sizes a multiple of 128).
 * Pair p = t·k + j routes token t to expert topk_ids[p].  Ids outside [0, E)
 * are dropped (not routed on this GPU).  Then
 *   counts[e]   = number of pairs routed to e
 *   offsets[e]  = Σ_{e' < e} ceil(counts[e'] / align) · align,  offsets[E] = M_total
 *   src_to_row[p] = offsets[e] + (number of pairs p' < p routed to e), or -1 if dropped
 *   row_to_src[r] = p for routed rows, -1 for padding rows and rows >= M_total
 * and, when xq is non-NULL, the permuted activations:
 *   a_out[r][:]   = xq[p / k][:]  (e4m3 codes, K bytes per row), 0 for padding rows
 *   sa_out[kb][r] = xs[kb][p / k] (1×128 scales, K-block-major), 0 for padding rows
 * Rows in [M_total, M_cap) of a_out/sa_out are not written.  If M_total > M_cap
 * (M_cap too small) no row at or beyond M_cap is written, a pair whose row would
 * be at or beyond M_cap gets src_to_row = -1 (dropped, so moe_combine never reads
 * past the GEMM output), and offsets[E] still reports M_total; the grouped GEMMs
 * called with M = M_cap stop at row M_cap.  M_cap = T·k + E·(align-1) is always
 * enough.
 *
 * topk_ids: [T][k] int32.  xq: [T][K] e4m3 codes or NULL (index-only mode).
 * xs: [K/128][T] fp32 (ignored when xq is NULL).  K % 128 == 0.
 * offsets [E+1], counts [E], src_to_row [T·k], row_to_src [M_cap] int32.
 * a_out [M_cap][K] bytes, sa_out [K/128][M_cap] fp32.
 * workspace: device scratch of at least fgg_moe_permute_workspace() bytes.
 * Limits: 1 <= E <= 1024, 1 <= k <= 64, align in {1..1024} (128 for the
 * GEMMs).  T == 0 writes offsets = 0 and nothing else.
 */
fgg_status fgg_moe_permute_workspace(int64_t T, int32_t k, int32_t E, size_t* bytes);
fgg_status fgg_moe_permute(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                           const void* xq, const float* xs, int64_t K, int32_t* offsets,
                           int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, void* a_out,
                           float* sa_out, int64_t M_cap, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * fgg_moe_permute_quantize — fgg_moe_permute with the activation quantization
 * fused into the gather.
 *
 * [MegaMoE] www.mqxn.cn/news/59821 §3 fuses the token quantization into the
 * dispatch; the rule is that of fgg_quantize_blockwise with {E4M3, F32, 1, 128}
 * ([DeepGEMM] §5.2: s = max|x| / 448 per 1x128 group, codes = round(x / s)).
 * x: [T][K] bf16 or fp32 token activations, row stride ldx >= K (elements),
 * 16-byte aligned rows.  Every output (offsets, counts, src_to_row,
 * row_to_src, a_out [M_cap][K] codes, sa_out [K/128][M_cap] scales) is
 * bit-identical to fgg_quantize_blockwise(x) followed by fgg_moe_permute with
 * its xq/xs; only the token-order codes are never materialised, and tokens
 * with no routed pair are not read.  Same limits, workspace and error rules
 * as fgg_moe_permute; x_dtype other than BF16/F32 is FGG_ERR_UNSUPPORTED.
 */
fgg_status fgg_moe_permute_quantize(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                    const void* x, fgg_dtype x_dtype, int64_t K, int64_t ldx,
                                    int32_t* offsets, int32_t* counts, int32_t* src_to_row,
                                    int32_t* row_to_src, void* a_out, float* sa_out, int64_t M_cap,
                                    void* workspace, size_t ws_bytes, void* stream);

/*
 * fgg_moe_permute_quantize_noalloc — fgg_moe_permute_quantize for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid allocation): the same arguments without the workspace, the same
 * outputs bit for bit, and no allocation by the library either.  The per-block
 * expert histograms live in a static device array of the library (2 MiB per
 * device, held until the process ends), so the call supports
 * ceil(T·k / 256) · E <= 524224 (T·k up to 4 193 792 pairs for E = 32, or
 * 130 816 for E = 1024) and returns FGG_ERR_UNSUPPORTED beyond that, before
 * launching anything.  Every call on a device uses that device's one array:
 * calls that overlap on one device (concurrent streams, or host threads
 * without ordering) race and must be serialized by the caller.  Nothing in the
 * array needs clearing between calls (every entry is written before it is read).
 */
fgg_status fgg_moe_permute_quantize_noalloc(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                            const void* x, fgg_dtype x_dtype, int64_t K, int64_t ldx,
                                            int32_t* offsets, int32_t* counts, int32_t* src_to_row,
                                            int32_t* row_to_src, void* a_out, float* sa_out, int64_t M_cap,
                                            void* stream);

/*
 * fgg_grouped_gemm_scaled — one launch for all groups (experts).
 *
 * The per-group formula of [Infra] Q "量化矩阵乘的维度和流程" with both
 * operands' scales applied to each K block inside the K loop and FP32
 * accumulation over all of K ([DeepGEMM] §2.2, §2.3):
 *   D[r][n] = bf16_rne( Σ_kb sA[r,kb] · sB[g,n,kb] · Σ_{k in kb} A[r][k] · B[g][n][k] )
 * with B stored [G][N][K] (the Q(W)ᵀ orientation of [W4A4] §1).
 *
 * FGG_LAYOUT_CONTIGUOUS (prefill): rows [offsets[g], offsets[g+1]) of A use
 *   expert g; M is the row count of A, sA and D (e.g. M_cap of the permute);
 *   every offsets[g] must be a multiple of 128 (moe_permute with align 128
 *   guarantees it).  Rows >= min(offsets[G], M) are not read or written
 *   (offsets[G] > M happens when the permute's M_cap was too small).  masked_m is optional here (NULL: every row of a segment is
 *   computed); when given, masked_m[g] (clamped to [0, segment length]) is
 *   group g's number of real rows, e.g. the permute's counts, and the rows
 *   [offsets[g] + masked_m[g], offsets[g+1]) are padding: not written, and
 *   their MFMA work is skipped in 16-row units (their A rows may still be
 *   read).  aq = {E4M3,F32,1,128}: a [M][K], a_scales [K/128][M];
 *   bq = {E4M3,F32,128,128}: b [G][N][K], b_scales [G][N/128][K/128].
 * FGG_LAYOUT_MASKED (decode, K >= 128): A is [G][M][K] (M = rows per group, <= 16);
 *   group g uses rows m < masked_m[g] (values clamped to [0, M]); other rows
 *   are neither read nor written.  aq = {E4M3,F32,1,128}: a_scales
 *   [G][K/128][M].  bq = {E2M1X2,E8M0,1,32}: b [G][N][K/2],
 *   b_scales [G][N][K/32] uint8 (the E8M0 scale multiplies each 32-element
 *   block inside the MFMA); or bq = {E2M1X2_TILED,E8M0,1,32}: the same weights
 *   re-laid out by fgg_pack_fp4_weights (b_scales 16-byte aligned), the same
 *   results bit for bit and a contiguous 1 KB per weight load; or
 *   bq = {E4M3,F32,128,128} as above.
 *   D is [G][M][ldd].
 * d: bf16, row stride ldd >= N.  N % 128 == 0, K % 128 == 0 (K == 0 gives zeros), 1 <= G <= 1024;
 * the contiguous layout supports K <= 16384.
 * Device-side values of offsets / masked_m are trusted within these rules.
 */
fgg_status fgg_grouped_gemm_scaled(fgg_layout layout, int32_t G, int64_t M, int64_t N, int64_t K,
                                   const void* a, const void* a_scales, fgg_qdesc aq,
                                   const void* b, const void* b_scales, fgg_qdesc bq,
                                   const int32_t* offsets, const int32_t* masked_m, void* d,
                                   int64_t ldd, void* stream);

/*
 * fgg_grouped_gemm_silu_quantize — the gate-up grouped GEMM (contiguous layout)
 * with SiLU(gate)·up and the 1x128 e4m3 requantization fused into its epilogue.
 *
 * [MegaMoE] §3.1 fuses the gate GEMM with its Swish activation so that the
 * intermediate never goes to memory; [Infra] Q "量化矩阵乘的维度和流程": the
 * next GEMM's input is quantized online.  B holds both projections of each
 * expert: b [G][2I][K] e4m3 (rows [0, I) gate, [I, 2I) up) with b_scales
 * [G][2I/128][K/128]; a, a_scales, offsets and their rules are those of
 * fgg_grouped_gemm_scaled CONTIGUOUS.  For every row r < offsets[G]:
 *   h[r][n] = Σ_kb sA[kb][r] · sB[g][n/128][kb] · Σ_{k in kb} A[r][k]·B[g][n][k]   (fp32, not rounded)
 *   a[r][c] = h[r][c] / (1 + e^-h[r][c]) · h[r][I + c]
 *   s_out[c/128][r] = max|a| / 448 over the 128 columns (1 if all are zero)
 *   q_out[r][c]     = e4m3_rne_satfinite(a · rcp(s))
 * All of this runs in fp32 on the accumulators with the hardware base-2
 * exponential and reciprocal (a few ulps each), so it is not the bit-exact rule
 * of fgg_quantize_blockwise (RNE of the IEEE quotient a / s): a value within a
 * few ulps of an e4m3 rounding midpoint may take the neighbouring code.  Against
 * the exact fp64 chain the scales agree to 2e-4 relative, >= 99.5 % of the codes
 * are equal, and each dequantized value lies within 2^-3·|a| + 2^-9·s +
 * 1e-2·(|a| + rms(a)) of the exact SiLU(gate)·up.
 * q_out is [M][I] bytes, s_out [I/128][M] fp32 (K-block-major, the activation
 * layout of the down GEMM).  Rows >= offsets[G] are not written.  counts
 * (optional, [G] int32) has the meaning of masked_m in fgg_grouped_gemm_scaled
 * CONTIGUOUS: padding rows past offsets[g] + counts[g] are not written.  The
 * separate path (bf16 H from fgg_grouped_gemm_scaled, then
 * fgg_quantize_blockwise with FGG_ACT_SILU_MUL) rounds H to bf16 first, so the
 * two may differ by one code where a value sits at a rounding boundary.
 * Requirements: I % 128 == 0, K % 128 == 0, K <= 16384, 1 <= G <= 1024.
 */
fgg_status fgg_grouped_gemm_silu_quantize(int32_t G, int64_t M, int64_t I, int64_t K, const void* a,
                                          const void* a_scales, fgg_qdesc aq, const void* b, const void* b_scales,
                                          fgg_qdesc bq, const int32_t* offsets, const int32_t* counts,
                                          void* q_out, float* s_out, void* stream);

/*
 * fgg_pack_fp4_weights — offline re-layout of FP4 expert weights for the masked
 * (decode) GEMM.
 *
 * [FP4MoE] "Blackwell架构下FP4 MoE模型的TFLOPS性能优化" §2.1: FP4 data should be
 * aligned to 128-bit boundaries and stored interleaved for the tensor-core path;
 * §3.1: a dedicated packed weight format.  The interleave chosen here is the
 * gfx950 MFMA operand order, so that one wave's load of one K block of 16 weight
 * rows is a contiguous 1 KB.  A pure byte permutation of
 *   b [G][N][K/2] (FGG_E2M1X2 codes) and b_scales [G][N][K/32] (E8M0):
 *   b_tiled: for g, nb = n / 16, kb = K block (128 elements, 64 bytes of a row),
 *     tile (g, nb, kb) is 1024 bytes at ((g·N/16 + nb)·(K/128) + kb)·1024; its
 *     16-byte piece 16c + r (c = 0..3, r = 0..15) holds row 16·nb + r, bytes
 *     [64·kb + 16·c, +16) of that row (K elements [128·kb + 32·c, +32)).
 *   s_tiled: for span j = 16 scale bytes of a row (4 K blocks), span (g, nb, j) is
 *     256 bytes at ((g·N/16 + nb)·ceil(K/512) + j)·256; bytes [16·r, 16·r + 16) hold
 *     row 16·nb + r's scale bytes [16·j, 16·j + 16), and 127 (2^0) past K/32.
 * Sizes from fgg_pack_fp4_weights_bytes: G·N·K/2 and G·(N/16)·ceil(K/512)·256 bytes.
 * Requires N % 16 == 0, K % 128 == 0 (else FGG_ERR_UNSUPPORTED); b, b_tiled and
 * s_tiled 16-byte aligned.  b_tiled / s_tiled must not overlap the inputs.
 */
fgg_status fgg_pack_fp4_weights_bytes(int32_t G, int64_t N, int64_t K, size_t* b_bytes, size_t* s_bytes);
fgg_status fgg_pack_fp4_weights(const void* b, const void* b_scales, int32_t G, int64_t N, int64_t K,
                                void* b_tiled, void* s_tiled, void* stream);

/*
 * fgg_scaled_gemm — the dense one-group case ([MegaMoE] §2.1 fp8_gemm with
 * fine-grained scales), and the W4A4 operator of [W4A4] §1.
 *
 * aq = {E4M3,F32,1,128}, bq = {E4M3,F32,128,128}: identical (bit for bit) to
 *   fgg_grouped_gemm_scaled(CONTIGUOUS, G = 1, offsets = {0, M}); any M >= 0
 *   (a partial last row block is handled).  epi must be NULL.
 * aq = bq = {E2M1X2,F32,1,16} (W4A4): a [M][K/2], a_scales [M][K/16];
 *   b [N][K/2], b_scales [N][K/16];
 *   D = bf16( Σ_g16 sA[m,g]·sB[n,g]·Σ_{k in g} A[m][k]·B[n][k]
 *             + (x_bf16 · l_down) · l_up + bias )
 *   The operands are dequantized once to fp16 (x·s rounded once) into the
 *   workspace and contracted with fp16 MFMA in fp32; the rank-32 intermediate
 *   x_bf16 · l_down is accumulated in fp32 (bf16 MFMA) and rounded to bf16.
 *   Range: fp16 holds magnitudes up to 65504, so every dequantized value
 *   |code · s| <= 6·s must fit: a 16-element group whose largest magnitude is
 *   at or above 65520 (s >= 10920) would become inf, and values below 2^-24
 *   flush to zero.  The call checks nothing of this on the device (it would
 *   need a pass over the scales); callers whose activations can leave the fp16
 *   range use the MXFP4 form below, whose E8M0 scales span 2^-127..2^127.
 * aq = bq = {E2M1X2,E8M0,1,32} (MXFP4 W4A4): a [M][K/2], a_scales [M][K/32]
 *   E8M0 bytes; b [N][K/2], b_scales [N][K/32]; the same epilogue:
 *   D = bf16( Σ_g32 2^(ea[m,g]-127)·2^(eb[n,g]-127)·Σ_{k in g} A[m][k]·B[n][k]
 *             + (x_bf16 · l_down) · l_up + bias )
 *   The E8M0 scales are applied by the FP4 matrix instruction itself (no
 *   dequantization, no promotion), fp32 accumulation; the rank-32 intermediate
 *   x_bf16 · l_down is rounded to bf16 as above.  Any M >= 0, N % 16 == 0,
 *   K % 128 == 0, 128 <= K <= 2^24, rank in {0, 32}; workspace (16-byte
 *   aligned) holds the [M][32] intermediate when rank is 32, else none.
 *   Requires M % 128 == 0, K % 128 == 0, 128 <= K <= 2^22, N % 128 == 0, rank in {0, 32}.
 *   workspace (256-byte aligned) must hold fgg_scaled_gemm_workspace() bytes:
 *   the fp16 copies of A and B, and with a low-rank branch the [M][32]
 *   intermediate.  The FP8 case needs none.
 */
fgg_status fgg_scaled_gemm_workspace(int64_t M, int64_t N, int64_t K, fgg_qdesc aq, fgg_qdesc bq,
                                     const fgg_epilogue* epi, size_t* bytes);
fgg_status fgg_scaled_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* a_scales,
                           fgg_qdesc aq, const void* b, const void* b_scales, fgg_qdesc bq,
                           const fgg_epilogue* epi, void* d, int64_t ldd, void* workspace,
                           size_t ws_bytes, void* stream);

/*
 * fgg_moe_combine — gate-weighted un-permute ([MegaMoE] §1 and §3: the
 * selected experts' outputs are summed with the gate weights).
 *   out[t][n] = bf16_rne( Σ_{j = 0..k-1, src_to_row[t·k+j] >= 0} w[t][j] · y[src_to_row[t·k+j]][n] )
 * summed in fp32 in increasing j (deterministic); a token with no routed slot
 * gets +0.
 * y: bf16 [rows][ldy]; src_to_row: [T·k] int32 (from moe_permute);
 * topk_w: [T][k] fp32; out: bf16 [T][ldo].  N % 8 == 0, ldy/ldo >= N and
 * multiples of 8.
 */
fgg_status fgg_moe_combine(const void* y, int64_t ldy, const int32_t* src_to_row,
                           const float* topk_w, int64_t T, int32_t k, int64_t N, void* out,
                           int64_t ldo, void* stream);

/*
 * fgg_moe_down_combine — the down projection and the gate-weighted combine in one
 * call.  [MegaMoE] §3 (Mega-MoE: the down GEMM, the weighting and the return to token
 * order in one pass) and [FP4MoE] §3.2 (results aggregated as they are produced): the
 * rows of tokens that have exactly one routed slot go from the GEMM's accumulators
 * straight to the token's output row.
 *
 * Result: out is bit-identical to
 *   fgg_grouped_gemm_scaled(CONTIGUOUS, G, M, N, K, a, a_scales, aq, b, b_scales, bq,
 *                           offsets, counts, y, ldy)
 *   fgg_moe_combine(y, ldy, src_to_row, topk_w, T, k, N, out, ldo)
 * For a routed row r whose token t has exactly one routed slot j, the GEMM's epilogue
 * writes out[t][n] = bf16_rne(fma(w[t][j], bf16_rne(y_fp32[r][n]), +0)) (the combine's
 * arithmetic for one slot) and leaves y[r] untouched; every other routed row is written
 * to y as by fgg_grouped_gemm_scaled, and the combine then handles only the tokens
 * with zero or at least two routed slots.
 *   aq = {E4M3,F32,1,128}, bq = {E4M3,F32,128,128}; a, a_scales, b, b_scales, offsets
 *     and the rules on G, M, N, K as fgg_grouped_gemm_scaled CONTIGUOUS;
 *   counts [G] (required): the per-expert routed rows from the permute;
 *   src_to_row [T·k], row_to_src [M] and topk_w [T][k]: the permute's maps (every
 *     row_to_src entry < T·k or -1) and the gate weights, as fgg_moe_combine;
 *   y bf16 [M][ldy] (rows of single-slot tokens are not written), out bf16 [T][ldo];
 *   workspace: ws_bytes >= fgg_moe_down_combine_workspace(M) (16-byte aligned), the
 *     per-row routing table the call writes and reads (roundup(M, 128) entries of 8 B).
 * The three kernels (routing table, GEMM, combine of the other tokens) run in order on
 * `stream`.  Errors as fgg_grouped_gemm_scaled; counts, the maps, the weights, y, out
 * and the workspace must be non-NULL.
 */
fgg_status fgg_moe_down_combine_workspace(int64_t M, size_t* bytes);
fgg_status fgg_moe_down_combine(int32_t G, int64_t M, int64_t N, int64_t K, const void* a,
                                const void* a_scales, fgg_qdesc aq, const void* b, const void* b_scales,
                                fgg_qdesc bq, const int32_t* offsets, const int32_t* counts,
                                const int32_t* src_to_row, const int32_t* row_to_src,
                                const float* topk_w, int64_t T, int32_t k, void* y, int64_t ldy,
                                void* workspace, size_t ws_bytes, void* out, int64_t ldo,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FGG_H_ */
