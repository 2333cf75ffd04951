/*
 * fp4.h -- C ABI of the MI355X (gfx950) microscaling FP4 library.
 *
 * What it computes
 *   Block-wise microscaling FP4 quantization along the contiguous (K) axis of a
 *   row-major [rows, cols] tensor, its dequantization and error sums, and the
 *   FP4 x FP4 block-scaled matrix product that consumes it, Y = A * B^T with
 *   fp32 accumulation.
 *
 *   MXFP4: blocks of 32 elements, E2M1 elements, one E8M0 (power-of-two) scale
 *          per block ("Bridging the Gap Between Promise and Performance for
 *          Microscaling FP4 Quantization", format definitions: G=32, E=FP4,
 *          S=E8M0).  Scale exponent = floor(log2(block amax)) - 2, clamped to
 *          [-127, 127] ("NVFP4 vs MXFP4: 4-Bit Floating Point for LLM Training
 *          and Inference (2026)", "A worked example, by hand").
 *   NVFP4: blocks of 16 elements, E2M1 elements, one E4M3 scale per block times
 *          one fp32 per-tensor scale ts = amax_tensor / (6 * 448) (same pages;
 *          NVFP4 vs MXFP4 Figure 2: global amax -> fp32 tensor scale -> block
 *          amax -> E4M3 -> E2M1 -> pack).
 *   Optional "micro-rotation": a block-diagonal Hadamard of the block size
 *          (Sylvester order, normalised by 1/sqrt(n)) applied to each block
 *          before quantization ("Bridging the Gap ...": rotations at the group
 *          level, Q(W H_k) Q(X H_k)^T, fused into activation quantization).
 *   Elements round to nearest-even on the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4,
 *   6}, saturating at +-6 (NVFP4 vs MXFP4, training recipe; "Microscaling
 *   Formats in Production LLM Inference", RTNE).  Two codes per byte, element
 *   2i in the low nibble; the code's sign bit is the sign of x / s.
 *
 * Conventions
 *   - Every pointer argument named x, y, codes, scales, global_scale, ws, sums
 *     and the GEMM operands is a DEVICE pointer (HIP device memory of the
 *     current device).  fp4_qconfig pointers are HOST pointers.
 *   - stream is a hipStream_t passed as void*; NULL means the default stream.
 *     All work is enqueued asynchronously on it; nothing synchronises.
 *   - The caller owns and allocates every buffer.  The library allocates no
 *     device memory and keeps no state between calls.  Workspaces may hold any
 *     contents on entry.
 *   - Calls that share a workspace must not overlap in time (same stream is
 *     enough).
 *   - Validation happens on the host before any launch: on error nothing is
 *     enqueued and a negative fp4_status is returned.  FP4_ERR_HIP reports a
 *     failed launch.
 *   - NaN and infinite inputs are outside the contract.
 */
#ifndef FP4_MI355X_H
#define FP4_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4_ABI_VERSION 5

typedef enum {
    FP4_OK = 0,
    FP4_ERR_INVALID_ARG = -1,   /* bad dims, leading dims, enum values, NULL */
    FP4_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement */
    FP4_ERR_ALIGNMENT = -3,     /* a pointer or leading dimension is misaligned */
    FP4_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required */
    FP4_ERR_HIP = -5,           /* a HIP launch failed */
    FP4_ERR_EXCHANGE = -6       /* FP4_GS_COMPUTE_ONE_PASS gave up its grid-wide wait
                                   (reported by callers that read the give-up flag) */
} fp4_status;

/* MXINT4 / NVINT4 ("Bridging the Gap ...", MXINT4 and NVINT4): the MXFP4 /
 * NVFP4 layouts with a 4-bit two's-complement integer element used
 * symmetrically (values -7 .. 7, nearest integer with ties to even, saturating;
 * the pattern 0x8 is never written).  MXINT4 keeps the E8M0 rule
 * floor(log2 amax) - 2; NVINT4 uses ts = amax / (7 * 448) and maps each block
 * maximum onto 7.  Only FP4_SCALE_ABSMAX applies to them. */
typedef enum {
    FP4_FMT_MXFP4 = 0,
    FP4_FMT_NVFP4 = 1,
    FP4_FMT_MXINT4 = 2,
    FP4_FMT_NVINT4 = 3
} fp4_format;
typedef enum {
    FP4_SCALE_ABSMAX = 0,       /* the block maximum sets the scale */
    FP4_SCALE_MSE = 1,          /* smallest block squared error in a window */
    FP4_SCALE_FOUR_OVER_SIX = 2 /* NVFP4: block maximum onto 6 or onto 4 */
} fp4_scale_rule;
typedef enum { FP4_DT_F32 = 0, FP4_DT_BF16 = 1 } fp4_dtype;
typedef enum { FP4_SCALES_ROWMAJOR = 0, FP4_SCALES_GEMM = 1 } fp4_scale_layout;
/* Layout of the packed codes (the same bytes, placed differently).  No page
 * fixes a storage order for the codes; the tiled one is this library's, for
 * weights that the GEMM streams from HBM.
 *   FP4_CODES_ROWMAJOR: byte b of row r (elements 2b, 2b + 1) at
 *     r * (cols / 2) + b.
 *   FP4_CODES_TILED: 8 KB tiles of 128 rows x 64 bytes (128 elements),
 *     row-major inside a tile; tile (r / 128, b / 64) starts at
 *     ((r / 128) * (cols / 128) + b / 64) * 8192, so byte b of row r is at
 *     that start + (r % 128) * 64 + b % 64.  rows and cols must be multiples
 *     of 128.  The GEMM's weight (B) operand then streams in whole 8 KB
 *     blocks instead of 64-byte pieces of rows far apart. */
typedef enum { FP4_CODES_ROWMAJOR = 0, FP4_CODES_TILED = 1 } fp4_code_layout;
/* OR'ed into the fmt of fp4_gemm / fp4_gemm_w4a16 (and their workspace
 * queries): b_codes are in the FP4_CODES_TILED layout (N % 128 == 0). */
#define FP4_GEMM_B_TILED 0x100
typedef enum {
    FP4_GS_COMPUTE = 0,          /* tensor scale from the tensor: maximum pass, then encode */
    FP4_GS_GIVEN = 1,            /* tensor scale read from *global_scale */
    FP4_GS_COMPUTE_ONE_PASS = 2  /* as FP4_GS_COMPUTE, both in one launch when it fits */
} fp4_gs_mode;

/* Quantization configuration (host struct).
 *   fmt           fp4_format.
 *   block         32 for MXFP4, 16 for NVFP4 (any other value is rejected).
 *   rotate        0, or equal to block: block Hadamard of that size first.
 *   rule          FP4_SCALE_ABSMAX: the block maximum sets the scale ("NVFP4 vs
 *                 MXFP4 ...", the worked example and Figure 2).
 *                 FP4_SCALE_MSE: the block-scale code with the smallest block
 *                 squared error among candidates around the absmax code c0
 *                 (MXFP4: c0, c0 + 1; NVFP4: c0 - 2 .. c0 + 6, tried in the
 *                 order c0, +1, -1, +2, -2, +3, +4, +5, +6 and kept within
 *                 0 .. 0x7E) ("Bridging the Gap ...", section 4.1: MR-GPTQ's
 *                 MSE-optimised scales; "NVFP4 vs MXFP4 ...": the best scale
 *                 does not always put the maximum on 6).
 *                 FP4_SCALE_FOUR_OVER_SIX (NVFP4 only, else
 *                 FP4_ERR_UNSUPPORTED): c0 or the code that maps the block
 *                 maximum onto 4, whichever has the smaller error ("NVFP4 vs
 *                 MXFP4 ...", follow-on research: Four Over Six).
 *                 The error of a candidate is summed in fp32 over the block in
 *                 element order, d = fl32(y - y^), acc = fma(d, d, acc), where
 *                 y^ is the value fp4_dequantize returns (in the rotated domain
 *                 when rotate != 0); a later candidate wins only with a
 *                 strictly smaller sum.  The NVFP4 tensor scale is the same
 *                 under every rule (amax / (6 * 448)). Blocks whose tensor
 *                 scale is 0 store zeros as under the absmax rule.
 *   scale_layout  FP4_SCALES_ROWMAJOR: byte (r, kb) at r * (cols/block) + kb.
 *                 FP4_SCALES_GEMM: the layout fp4_gemm reads; byte positions
 *                 are given by fp4_scale_offset.  For NVFP4 the two layouts
 *                 coincide.
 *   rounding      FP4_ROUND_NEAREST (ties to even), or FP4_ROUND_STOCHASTIC
 *                 ("NVFP4 vs MXFP4 ...", the training recipe: up or down with
 *                 probability proportional to proximity, so the expected value
 *                 is the input) for E2M1 elements with FP4_SCALE_ABSMAX: the
 *                 quotient a = min(|q|, 6) between grid neighbours lo < a < hi
 *                 rounds up when u < (a - lo) / (hi - lo), with u = (w >> 8) *
 *                 2^-24 and w word e % 4 of Philox4x32-10 (Salmon et al.,
 *                 SC'11) at counter (e / 4 low 32 bits, high 32 bits, 0, 0)
 *                 and key (seed[0], seed[1]), e = r * cols + c the element.
 *   block_rows    0 or 1: blocks along a row.  16 (NVFP4, rotate 0,
 *                 FP4_SCALE_ABSMAX): each 16 x 16 tile (16 rows x one 16-column
 *                 block) takes its scale from the tile maximum, stored in the
 *                 scale byte of each of its rows ("NVFP4 vs MXFP4 ...",
 *                 two-dimensional weight scaling: a tile and its transpose
 *                 share the scale).  A last tile of fewer rows uses those rows.
 *   rot_signs     sign diagonal of the rotation: bit i of the 128-bit mask
 *                 (word i / 32, bit i % 32) negates element i of each rotation
 *                 group before the Hadamard (a randomised Hadamard transform,
 *                 "Microscaling Formats in Production ...", orthogonal
 *                 rotations); all zero is the plain transform.  The inverse
 *                 (fp4_dequantize, fp4_error_sums) applies it after.
 *   seed          stochastic-rounding key.
 *   code_layout   fp4_code_layout of the codes that fp4_quantize writes and
 *                 fp4_dequantize / fp4_error_sums read.
 * rotate may also be 64 or 128 for MXFP4 / MXINT4 ("Bridging the Gap ...":
 * larger rotations help MXFP4): rotation groups of 2 or 4 blocks, cols a
 * multiple of rotate; scales stay per 32-element block. */
typedef enum { FP4_ROUND_NEAREST = 0, FP4_ROUND_STOCHASTIC = 1 } fp4_rounding;
typedef struct {
    int32_t fmt;
    int32_t block;
    int32_t rotate;
    int32_t rule;
    int32_t scale_layout;
    int32_t rounding;
    int32_t block_rows;
    uint32_t rot_signs[4];
    uint32_t seed[2];
    int32_t code_layout;
} fp4_qconfig;

/* ---------------------------------------------------------------- sizes */

/* Bytes of packed codes for [rows, cols]: rows * cols / 2, two 4-bit codes per
 * byte ("NVFP4 vs MXFP4 ...", Figure 2: E2M1 values packed two per byte), in
 * either code layout.  0 for negative sizes or odd cols.  Host function. */
size_t fp4_codes_bytes(int64_t rows, int64_t cols);

/* Bytes of the scale array, including the padding of the GEMM layout
 * (MXFP4 GEMM layout pads rows to 32 and cols to 256).  0 on invalid input.
 * Unpadded sizes give 4.25 (MXFP4) and 4.5 (NVFP4) bits per element together
 * with the codes ("NVFP4 vs MXFP4", storage overhead).  Host function. */
size_t fp4_scales_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols);

/* Workspace bytes fp4_quantize and fp4_global_scale need (NVFP4 and NVINT4:
 * 8192 bytes; MXFP4 and MXINT4: 0).  Bytes [0, 2048) hold the partial maxima
 * of the global-amax pass (any contents); bytes [4096, 8192) are the exchange
 * region of FP4_GS_COMPUTE_ONE_PASS (see fp4_quantize).  Host function. */
size_t fp4_workspace_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols);

/* Zero-fill ws_bytes of device workspace on the stream (a kernel, so it may be
 * captured in a graph): the preparation the single-pass exchange region needs
 * before its first use (FP4_GS_COMPUTE_ONE_PASS).  Requirements: ws 8-byte
 * aligned, ws_bytes a multiple of 4.  Asynchronous; FP4_ERR_INVALID_ARG for
 * NULL or zero bytes. */
int fp4_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Byte index inside the scale array of the scale of (row r, block kb), for the
 * layout named in cfg; -1 if out of range.  The GEMM layout is this library's
 * own scale reordering for the matrix-core loads ("Portable FP4 Quantization
 * for Heterogeneous Accelerators", section 2.4: scales reordered to the
 * layout the GEMM's loads want); this function is its definition for
 * callers and tests.  Host function. */
int64_t fp4_scale_offset(const fp4_qconfig* cfg, int64_t rows, int64_t cols,
                         int64_t r, int64_t kb);

/* ------------------------------------------------------------- quantize */

/* Quantize x [rows, cols] (row-major, leading dimension ldx elements, element
 * type xdt) into codes [rows, cols/2] (dense) and scales (layout of cfg).
 *   NVFP4: gs_mode FP4_GS_COMPUTE computes ts = amax(|x'|)/2688 over the whole
 *   [rows, cols] tensor (x' = the rotated tensor when rotate != 0) and writes
 *   it to *global_scale; FP4_GS_GIVEN reads ts from *global_scale.  A block
 *   whose scale (e4m3 * ts) is zero stores all-zero codes.
 *   FP4_GS_COMPUTE_ONE_PASS gives the same codes, scales and ts as
 *   FP4_GS_COMPUTE, reading x once: for bf16 input without 16x16 blocks, when
 *   the tensor fits one workgroup per CU at 16 x 8 x 1024 elements per
 *   workgroup (about 32 M elements on 256 CUs), a single launch takes the
 *   maximum, exchanges it across the grid and encodes from registers;
 *   otherwise it runs the two passes of FP4_GS_COMPUTE.  Its grid waits for
 *   all of its workgroups, so no other FP4_GS_COMPUTE_ONE_PASS call (nor any
 *   other kernel that waits for a whole grid) may run on the device at the
 *   same time; a wait that outlasts a few seconds gives up: the codes of the
 *   workgroups that gave up are zero, NaN is written to *global_scale and the
 *   32-bit word at byte 4100 of ws (the give-up flag) becomes non-zero.  The
 *   call still returns FP4_OK (it cannot wait for the kernel); a caller that
 *   needs to know synchronises and reads the flag, and reports
 *   FP4_ERR_EXCHANGE.  Bytes [4096, 8192) of ws must be zero before the first
 *   call that uses this ws (every call leaves them ready for the next; after
 *   a give-up they need zeroing again; fp4_workspace_init does it); ws
 *   8-byte aligned.
 *   MXFP4 ignores global_scale and gs_mode (global_scale may be NULL).
 * ws/ws_bytes: device workspace of fp4_workspace_bytes() bytes, any contents
 * except as above (needed only by NVFP4 with a computed scale; may be NULL
 * otherwise).
 * Requirements: rows >= 0, cols >= 0, cols % block == 0, ldx >= cols, x
 * 16-byte aligned and ldx * sizeof(xdt) a multiple of 16 (when rows > 1),
 * codes 16-byte aligned.  rows == 0 or cols == 0 is a no-op (for NVFP4 with
 * FP4_GS_COMPUTE, ts = 0 is written). */
int fp4_quantize(const fp4_qconfig* cfg, const void* x, int32_t xdt,
                 int64_t rows, int64_t cols, int64_t ldx,
                 uint8_t* codes, uint8_t* scales, float* global_scale, int32_t gs_mode,
                 void* ws, size_t ws_bytes, void* stream);

/* 1 when fp4_quantize with FP4_GS_COMPUTE_ONE_PASS would quantize this
 * configuration and shape in one launch on the current device, 0 when it
 * would fall back to the two passes (MX formats, fp32 input, 16x16 blocks,
 * misaligned rows, tensors past the one-launch capacity) or on any error.
 * Host function; it queries the device's CU count once. */
int fp4_quantize_one_pass_fits(const fp4_qconfig* cfg, int32_t xdt, int64_t rows, int64_t cols,
                               int64_t ldx);

/* NVFP4 per-tensor scale only: writes ts = amax(|x'|) / 2688 to
 * *global_scale (x' = the rotated tensor when cfg->rotate != 0), exactly as
 * fp4_quantize does with FP4_GS_COMPUTE, which is this call followed by
 * fp4_quantize with FP4_GS_GIVEN.  For callers that fix the tensor scale once
 * (static scales) or schedule the two passes themselves.  Same workspace and
 * argument rules as fp4_quantize; MXFP4 configurations are rejected with
 * FP4_ERR_INVALID_ARG. */
int fp4_global_scale(const fp4_qconfig* cfg, const void* x, int32_t xdt,
                     int64_t rows, int64_t cols, int64_t ldx, float* global_scale,
                     void* ws, size_t ws_bytes, void* stream);

/* fp4_quantize without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc.  The same computation and results as
 * fp4_quantize with the same arguments; the NVFP4 / NVINT4 scratch (partial
 * maxima, single-pass exchange region) is a static device array of 8192
 * bytes inside the library, one per GPU, held until the process ends.  The
 * call allocates nothing; its first call on a device also zeroes the exchange
 * region (a fill kernel on `stream`).  Every call on a GPU uses that GPU's one
 * array, which keeps the last call's contents: calls that may overlap in time
 * on one GPU (other streams, other host threads) race on it and must be
 * serialised by the caller (one stream is enough).  With
 * FP4_GS_COMPUTE_ONE_PASS a one-workgroup kernel is queued before the
 * quantization that zeroes the exchange region if an earlier call gave up
 * its grid-wide wait (NaN tensor scale; the region then needs zeroing, which
 * a caller cannot do for the static array).  Returns
 * FP4_ERR_WORKSPACE if a configuration would need more than the static
 * scratch (none does today), otherwise exactly what fp4_quantize returns. */
int fp4_quantize_noalloc(const fp4_qconfig* cfg, const void* x, int32_t xdt,
                         int64_t rows, int64_t cols, int64_t ldx,
                         uint8_t* codes, uint8_t* scales, float* global_scale, int32_t gs_mode,
                         void* stream);

/* One quantization of a batch: the arguments of fp4_quantize. */
typedef struct {
    fp4_qconfig cfg;
    const void* x;
    int32_t xdt;
    int64_t rows;
    int64_t cols;
    int64_t ldx;
    uint8_t* codes;
    uint8_t* scales;
    float* global_scale;
    int32_t gs_mode;
} fp4_quant_job;

/* Workspace bytes of fp4_quantize_batch for n jobs: 2048 per job.  Host
 * function. */
size_t fp4_quantize_batch_workspace_bytes(int32_t n);

/* n independent quantizations, each exactly as fp4_quantize defines it (the
 * same codes, scales and tensor scale as n fp4_quantize calls), in few
 * launches.  Jobs with bf16 input, absmax block scales, nearest rounding,
 * one-row blocks and no rotation or the block-sized one share two launches
 * of one kernel: the first holds every MXFP4 / MXINT4 job, every NVFP4 /
 * NVINT4 job with its tensor scale given and the tensor-maximum pass of the
 * NVFP4 / NVINT4 jobs that compute it; the second encodes those jobs (up to 16
 * jobs per launch and 64 per launch pair; more make more launches).  Each
 * tensor then pays one share of a launch's ramp-up and drain instead of a
 * whole one.  Other jobs (other configurations, fp32 input, empty tensors)
 * run as their own fp4_quantize launches, in job order among themselves.  An NVFP4 / NVINT4 job with
 * FP4_GS_COMPUTE_ONE_PASS runs as FP4_GS_COMPUTE (same results; no exchange
 * region involved).
 * jobs: host array of n jobs, read during the call only; each job follows
 *   fp4_quantize's argument rules.  No job's outputs may overlap another
 *   job's input or outputs.
 * ws/ws_bytes: device workspace of fp4_quantize_batch_workspace_bytes(n)
 *   bytes, 4-byte aligned, any contents (job i uses bytes [2048 i,
 *   2048 i + 2048) when it computes its tensor scale); may be NULL when no
 *   job computes one.
 * Every job is checked before anything is launched: the first failing job's
 * status is returned and nothing runs.  n == 0 is a no-op; n < 0, or
 * jobs == NULL with n > 0, is FP4_ERR_INVALID_ARG.  Asynchronous on stream. */
int fp4_quantize_batch(int32_t n, const fp4_quant_job* jobs, void* ws, size_t ws_bytes,
                       void* stream);

/* ----------------------------------------------------------- dequantize */

/* y [rows, cols] (leading dimension ldy, element type ydt) =
 *   MXFP4: e2m1 * 2^(c - 127);  NVFP4: fl32(fl32(e2m1 * e4m3) * ts),
 * then, if inverse_rotate != 0 and cfg->rotate != 0, the block Hadamard again
 * (it is its own inverse), giving values in the original domain.  bf16 output
 * rounds to nearest-even.  Scales and codes are read in cfg's layouts. */
int fp4_dequantize(const fp4_qconfig* cfg, const uint8_t* codes, const uint8_t* scales,
                   const float* global_scale, int64_t rows, int64_t cols,
                   void* y, int32_t ydt, int64_t ldy, int32_t inverse_rotate, void* stream);

/* Error sums of the quantization of x ("Portable FP4 Quantization for
 * Heterogeneous Accelerators", section 3.2: NMSE and cosine similarity):
 *   sums[0] = sum (x - x^)^2, sums[1] = sum x^2, sums[2] = sum x * x^,
 *   sums[3] = sum x^^2, in double, over all rows x cols elements, where x^ is
 *   the dequantized value brought back to the original domain (inverse
 *   rotation when cfg->rotate != 0).  sums is a device array of 4 doubles.
 *   ws: device workspace of fp4_error_workspace_bytes() bytes (any contents).
 *   The reduction order is fixed, so the sums are deterministic. */
size_t fp4_error_workspace_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols);
int fp4_error_sums(const fp4_qconfig* cfg, const void* x, int32_t xdt,
                   int64_t rows, int64_t cols, int64_t ldx,
                   const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                   double* sums, void* ws, size_t ws_bytes, void* stream);

/* Re-lay scales from FP4_SCALES_ROWMAJOR [rows, cols/block] into
 * FP4_SCALES_GEMM (padding bytes are written as 127, i.e. scale 1, and are
 * never used by fp4_gemm).  For weights quantized elsewhere.  MXFP4 only:
 * for NVFP4 the two layouts coincide and FP4_ERR_UNSUPPORTED is returned. */
int fp4_scales_to_gemm_layout(const fp4_qconfig* cfg, const uint8_t* rowmajor,
                              int64_t rows, int64_t cols, uint8_t* gemm_scales, void* stream);

/* ----------------------------------------------------------------- GEMM */

/* Y[M, N] = sum_k A[m, k] * B[n, k] ("Bridging the Gap ...": the kernels
 * compute Q(W H_k) Q(X H_k)^T; "NVFP4 vs MXFP4", hardware execution: block
 * scales applied inside the product, higher-precision accumulation).
 *   A: a_codes [M, K/2] dense, a_scales in FP4_SCALES_GEMM layout for (M, K).
 *   B: b_codes [N, K/2] dense, b_scales in FP4_SCALES_GEMM layout for (N, K).
 *   fmt | FP4_GEMM_B_TILED: b_codes in the FP4_CODES_TILED layout (N % 128
 *   == 0, else FP4_ERR_INVALID_ARG); the result is bit-identical to the
 *   row-major call.
 *   NVFP4: a_gs / b_gs point to the fp32 per-tensor scales (device); the
 *   product is multiplied by (*a_gs) * (*b_gs).  MXFP4 ignores them.
 *   Accumulation is fp32.  y has leading dimension ldy >= N and type ydt
 *   (bf16 rounds to nearest-even).  The GEMM does not rotate: the caller
 *   quantizes both operands with the same rotation setting.
 * ws/ws_bytes: device workspace of fp4_gemm_workspace_bytes() bytes (any
 * contents; used for split-K partial sums; 16-byte aligned).
 * MXINT4 / NVINT4 operands: the same call with fmt = FP4_FMT_MXINT4 (GEMM-
 * layout E8M0 scales; n * 2^e expanded exactly to bf16, bf16 MFMA; exact for
 * every operand fp4_quantize writes -- scale codes up to 252 with elements
 * -7 .. 7 -- and for any element with codes up to 251: the element -8 at
 * code 252, or any code above 252, leaves bf16's range) or
 * FP4_FMT_NVINT4 (n * e4m3 expanded exactly to fp16, fp16 MFMA, tensor scales
 * in the epilogue); K % 256 == 0 for them.
 * Requirements: M, N >= 0, K >= 0 with K % 128 == 0; codes and scales
 * 16-byte aligned (both stream into LDS in 16-byte pieces). */
size_t fp4_gemm_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K);
int fp4_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K,
             const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gs,
             void* y, int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/* Weight-only GEMM (W4A16): Y[M, N] = sum_k A[m, k] * dequant(B)[n, k]
 * ("Bridging the Gap ...": the W4A16 control, 16-bit activations times FP4
 * weights; decode, where the weights stream from HBM once per token, is the
 * serving case the pages emphasise).
 *   A: bf16 activations [M, K], row stride lda (elements), unquantized.
 *   B: b_codes [N, K/2] dense (fmt | FP4_GEMM_B_TILED: the FP4_CODES_TILED
 *      layout, N % 128 == 0), b_scales in FP4_SCALES_GEMM layout for (N, K)
 *      (NVFP4: row-major), b_gs the NVFP4 tensor scale (device fp32; MXFP4
 *      ignores it).  MXINT4 / NVINT4 weights take the same call (the integer
 *      element times its scale is exact in bf16).  B is dequantized exactly (e2m1 * scale is exact in bf16)
 *      and multiplied on bf16 MFMA with fp32 accumulation.
 *   No rotation is applied: a caller that quantized B with the block
 *   Hadamard passes activations rotated the same way.
 * ws/ws_bytes: device workspace of fp4_gemm_w4a16_workspace_bytes() bytes
 * (any contents, 16-byte aligned; split-K partial sums; without it the call
 * runs unsplit).
 * Requirements: M, N >= 0, K >= 0 with K % 256 == 0; lda >= K; a, b_codes and
 * b_scales 16-byte aligned, lda * 2 a multiple of 16 (when M > 1). */
size_t fp4_gemm_w4a16_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K);
int fp4_gemm_w4a16(int32_t fmt, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                   const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gs,
                   void* y, int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- misc */

const char* fp4_status_str(int status);
int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_H */
