// api.cpp -- the C ABI declared in include/fp4.h: host-side validation, size
// and layout helpers, and dispatch to the gfx950 kernels.  Nothing here
// touches the GPU before every argument has been checked.
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "fp4.h"
#include "fp4_device.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_bytes(int32_t dt) { return dt == FP4_DT_F32 ? 4 : (dt == FP4_DT_BF16 ? 2 : 0); }

// Returns FP4_OK when cfg describes a supported quantization of [rows, cols].
int check_cfg(const fp4_qconfig* cfg, int64_t rows, int64_t cols) {
  if (!cfg) return FP4_ERR_INVALID_ARG;
  if (cfg->fmt < FP4_FMT_MXFP4 || cfg->fmt > FP4_FMT_NVINT4) return FP4_ERR_INVALID_ARG;
  const int G = fp4k::fmt_block(cfg->fmt);
  if (cfg->block != G) return FP4_ERR_INVALID_ARG;
  const bool big_rot = fp4k::fmt_mx(cfg->fmt) && (cfg->rotate == 64 || cfg->rotate == 128);
  if (cfg->rotate != 0 && cfg->rotate != G && !big_rot) return FP4_ERR_INVALID_ARG;
  if (cfg->rule != FP4_SCALE_ABSMAX && cfg->rule != FP4_SCALE_MSE &&
      cfg->rule != FP4_SCALE_FOUR_OVER_SIX)
    return FP4_ERR_INVALID_ARG;
  if (cfg->rule == FP4_SCALE_FOUR_OVER_SIX && cfg->fmt != FP4_FMT_NVFP4) return FP4_ERR_UNSUPPORTED;
  if (cfg->rule != FP4_SCALE_ABSMAX && fp4k::fmt_int(cfg->fmt)) return FP4_ERR_UNSUPPORTED;
  if (cfg->scale_layout != FP4_SCALES_ROWMAJOR && cfg->scale_layout != FP4_SCALES_GEMM)
    return FP4_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || cols % G != 0) return FP4_ERR_INVALID_ARG;
  if (cfg->code_layout != FP4_CODES_ROWMAJOR && cfg->code_layout != FP4_CODES_TILED)
    return FP4_ERR_INVALID_ARG;
  if (cfg->code_layout == FP4_CODES_TILED && (rows % 128 != 0 || cols % 128 != 0))
    return FP4_ERR_INVALID_ARG;
  if (cfg->rotate != 0 && cols % cfg->rotate != 0) return FP4_ERR_INVALID_ARG;
  if (cfg->rounding != FP4_ROUND_NEAREST && cfg->rounding != FP4_ROUND_STOCHASTIC)
    return FP4_ERR_INVALID_ARG;
  if (cfg->rounding == FP4_ROUND_STOCHASTIC &&
      (fp4k::fmt_int(cfg->fmt) || cfg->rule != FP4_SCALE_ABSMAX))
    return FP4_ERR_UNSUPPORTED;
  if (cfg->block_rows != 0 && cfg->block_rows != 1 && cfg->block_rows != 16)
    return FP4_ERR_INVALID_ARG;
  if (cfg->block_rows == 16 &&
      (cfg->fmt != FP4_FMT_NVFP4 || cfg->rotate != 0 || cfg->rule != FP4_SCALE_ABSMAX))
    return FP4_ERR_UNSUPPORTED;
  // 32-bit block indexing inside the kernels
  if (rows >= (int64_t)1 << 31 || cols >= (int64_t)1 << 31 || rows * cols >= ((int64_t)1 << 32))
    return FP4_ERR_UNSUPPORTED;
  return FP4_OK;
}

int check_ld(const void* p, int32_t dt, int64_t rows, int64_t cols, int64_t ld) {
  const int eb = dtype_bytes(dt);
  if (eb == 0) return FP4_ERR_INVALID_ARG;
  if (ld < cols) return FP4_ERR_INVALID_ARG;
  if (rows > 0 && cols > 0) {
    if (!p) return FP4_ERR_INVALID_ARG;
    if (!aligned16(p)) return FP4_ERR_ALIGNMENT;
    if (rows > 1 && (ld * eb) % 16 != 0) return FP4_ERR_ALIGNMENT;
  }
  return FP4_OK;
}

// Rotation group in blocks (0: no rotation).
int rot_blocks(const fp4_qconfig* cfg) { return cfg->rotate / cfg->block; }

fp4k::QParams qparams(const fp4_qconfig* cfg, int64_t cols) {
  fp4k::QParams P{};
  for (int i = 0; i < 4; ++i) P.signs[i] = cfg->rot_signs[i];
  P.any_sign = (cfg->rot_signs[0] | cfg->rot_signs[1] | cfg->rot_signs[2] | cfg->rot_signs[3]) != 0u;
  if (cfg->rotate == 16) {  // a 16-point group: only the low 16 bits are positions
    P.signs[0] &= 0xFFFFu;
    P.any_sign = P.signs[0] != 0u;
  }
  if (cfg->rotate == 32) P.any_sign = P.signs[0] != 0u;
  if (cfg->rotate == 64) P.any_sign = (P.signs[0] | P.signs[1]) != 0u;
  P.seed0 = cfg->seed[0];
  P.seed1 = cfg->seed[1];
  P.tiled = cfg->code_layout == FP4_CODES_TILED ? 1u : 0u;
  P.cols = cols;
  return P;
}

bool gemm_layout(const fp4_qconfig* cfg) {
  return fp4k::fmt_mx(cfg->fmt) && cfg->scale_layout == FP4_SCALES_GEMM;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

// NVFP4 workspace: bytes [0, 2048) one fp32 partial maximum per workgroup of
// the amax pass (any contents); bytes [4096, 8192) the exchange region of the
// single-pass kernel (a call number, then one 64-bit slot per workgroup).
constexpr size_t kNvWorkspace = 8192;
constexpr size_t kNvExchange = 4096;
constexpr int kNvExchangeSlots = (int)((kNvWorkspace - kNvExchange - 64) / 8);
// Batch workspace per job: the partial maxima of its tensor-scale pass.
constexpr size_t kBatchJobWorkspace = 2048;

// fp4_quantize's argument checks, apart from the workspace.
int check_quantize(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows, int64_t cols,
                   int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                   const float* global_scale, int32_t gs_mode) {
  int rc = check_cfg(cfg, rows, cols);
  if (rc != FP4_OK) return rc;
  rc = check_ld(x, xdt, rows, cols, ldx);
  if (rc != FP4_OK) return rc;
  if (rows != 0 && cols != 0) {
    if (!codes || !scales) return FP4_ERR_INVALID_ARG;
    if (!aligned16(codes)) return FP4_ERR_ALIGNMENT;
  }
  if (fp4k::fmt_mx(cfg->fmt)) return FP4_OK;
  if (gs_mode != FP4_GS_COMPUTE && gs_mode != FP4_GS_GIVEN && gs_mode != FP4_GS_COMPUTE_ONE_PASS)
    return FP4_ERR_INVALID_ARG;
  if (!global_scale) return FP4_ERR_INVALID_ARG;
  return FP4_OK;
}

int quantize_mx(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows, int64_t cols,
                int64_t ldx, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return FP4_OK;
  return hip_status(fp4lib::launch_quantize_mx(cfg->fmt, x, xdt, rot_blocks(cfg), cfg->rule,
                                               cfg->rounding, rows, cols, ldx, codes, scales,
                                               gemm_layout(cfg) ? 1 : 0, qparams(cfg, cols), st));
}

// NVFP4 / NVINT4 in two passes: with partials (room for 512 floats) the
// tensor-maximum pass first, then the encoding; without, the encoding with
// the tensor scale read from *global_scale.
int quantize_nv_passes(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows,
                       int64_t cols, int64_t ldx, uint8_t* codes, uint8_t* scales,
                       float* global_scale, float* partials, hipStream_t st) {
  const bool empty = rows == 0 || cols == 0;
  int npart = 0;
  if (partials) {
    if (empty) return hip_status(fp4lib::launch_amax_final(cfg->fmt, nullptr, 0, global_scale, st));
    npart = fp4lib::amax_partials(rows, cols, cfg->rotate != 0, xdt);
    hipError_t e = fp4lib::launch_amax_nv(x, xdt, cfg->rotate != 0, qparams(cfg, cols).signs[0],
                                          rows, cols, ldx, partials, npart, st);
    if (e != hipSuccess) return FP4_ERR_HIP;
  }
  if (empty) return FP4_OK;
  return hip_status(fp4lib::launch_quantize_nv(cfg->fmt, x, xdt, cfg->rotate != 0, cfg->rule,
                                               cfg->rounding, cfg->block_rows, rows, cols, ldx,
                                               codes, scales, global_scale, partials, npart,
                                               qparams(cfg, cols), st));
}

// Jobs that the grouped launches take (see fp4_quantize_batch).
bool batch_mergeable(const fp4_quant_job& j) {
  const fp4_qconfig& c = j.cfg;
  return j.xdt == FP4_DT_BF16 && j.rows > 0 && j.cols > 0 && c.rule == FP4_SCALE_ABSMAX &&
         c.rounding == FP4_ROUND_NEAREST && c.block_rows <= 1 &&
         (c.rotate == 0 || c.rotate == c.block);
}

}  // namespace

extern "C" {

int fp4_abi_version(void) { return FP4_ABI_VERSION; }

const char* fp4_status_str(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_INVALID_ARG: return "invalid argument";
    case FP4_ERR_UNSUPPORTED: return "unsupported";
    case FP4_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case FP4_ERR_WORKSPACE: return "workspace missing or too small";
    case FP4_ERR_HIP: return "HIP launch failed";
    case FP4_ERR_EXCHANGE: return "single-pass exchange wait gave up";
    default: return "unknown status";
  }
}

size_t fp4_codes_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || cols % 2 != 0) return 0;
  return (size_t)(rows * (cols / 2));
}

size_t fp4_scales_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols) {
  if (check_cfg(cfg, rows, cols) != FP4_OK) return 0;
  if (gemm_layout(cfg)) return (size_t)(((rows + 31) / 32) * fp4k::mx_gemm_kchunks(cols) * 256);
  return (size_t)(rows * (cols / cfg->block));
}

size_t fp4_workspace_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols) {
  if (check_cfg(cfg, rows, cols) != FP4_OK) return 0;
  return fp4k::fmt_mx(cfg->fmt) ? 0 : kNvWorkspace;
}

int64_t fp4_scale_offset(const fp4_qconfig* cfg, int64_t rows, int64_t cols, int64_t r, int64_t kb) {
  if (check_cfg(cfg, rows, cols) != FP4_OK) return -1;
  const int64_t nb = cols / cfg->block;
  if (r < 0 || r >= rows || kb < 0 || kb >= nb) return -1;
  if (gemm_layout(cfg)) return fp4k::mx_gemm_scale_offset(r, kb, fp4k::mx_gemm_kchunks(cols));
  return r * nb + kb;
}

int fp4_quantize(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows, int64_t cols,
                 int64_t ldx, uint8_t* codes, uint8_t* scales, float* global_scale,
                 int32_t gs_mode, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_quantize(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, gs_mode);
  if (rc != FP4_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fp4k::fmt_mx(cfg->fmt)) return quantize_mx(cfg, x, xdt, rows, cols, ldx, codes, scales, st);
  float* partials = nullptr;
  if (gs_mode != FP4_GS_GIVEN) {
    if (!ws || ws_bytes < fp4_workspace_bytes(cfg, rows, cols)) return FP4_ERR_WORKSPACE;
    const uintptr_t amask = gs_mode == FP4_GS_COMPUTE_ONE_PASS ? 7u : 3u;  // 64-bit slots
    if ((reinterpret_cast<uintptr_t>(ws) & amask) != 0) return FP4_ERR_ALIGNMENT;
    if (gs_mode == FP4_GS_COMPUTE_ONE_PASS && rows != 0 && cols != 0) {
      uint32_t* xchg = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kNvExchange);
      const hipError_t e = fp4lib::launch_quantize_nv_one_pass(
          cfg->fmt, x, xdt, cfg->rotate != 0, cfg->rule, cfg->rounding, cfg->block_rows, rows, cols,
          ldx, codes, scales, global_scale, xchg, kNvExchangeSlots, qparams(cfg, cols), st);
      if (e != hipErrorNotSupported) return hip_status(e);
    }
    partials = static_cast<float*>(ws);
  }
  return quantize_nv_passes(cfg, x, xdt, rows, cols, ldx, codes, scales, global_scale, partials, st);
}

size_t fp4_quantize_batch_workspace_bytes(int32_t n) {
  return n > 0 ? (size_t)n * kBatchJobWorkspace : 0;
}

int fp4_quantize_batch(int32_t n, const fp4_quant_job* jobs, void* ws, size_t ws_bytes,
                       void* stream) {
  if (n < 0) return FP4_ERR_INVALID_ARG;
  if (n == 0) return FP4_OK;
  if (!jobs) return FP4_ERR_INVALID_ARG;
  bool need_ws = false;
  for (int32_t i = 0; i < n; ++i) {
    const fp4_quant_job& j = jobs[i];
    const int rc = check_quantize(&j.cfg, j.x, j.xdt, j.rows, j.cols, j.ldx, j.codes, j.scales,
                                  j.global_scale, j.gs_mode);
    if (rc != FP4_OK) return rc;
    if (!fp4k::fmt_mx(j.cfg.fmt) && j.gs_mode != FP4_GS_GIVEN) need_ws = true;
  }
  if (need_ws) {
    if (!ws || ws_bytes < fp4_quantize_batch_workspace_bytes(n)) return FP4_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return FP4_ERR_ALIGNMENT;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // grouped jobs are launched kBatchChunk at a time (no host allocation)
  constexpr int kBatchChunk = 64;
  fp4lib::BatchItem items[kBatchChunk];
  int nitems = 0;
  for (int32_t i = 0; i < n; ++i) {
    const fp4_quant_job& j = jobs[i];
    const bool mx = fp4k::fmt_mx(j.cfg.fmt);
    float* part = !mx && j.gs_mode != FP4_GS_GIVEN
                      ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + i * kBatchJobWorkspace)
                      : nullptr;
    if (batch_mergeable(j)) {
      fp4lib::BatchItem it{};
      it.fmt = j.cfg.fmt;
      it.rotate = j.cfg.rotate != 0 ? 1 : 0;
      it.gemm_layout = gemm_layout(&j.cfg) ? 1 : 0;
      it.x = j.x;
      it.rows = j.rows;
      it.cols = j.cols;
      it.ldx = j.ldx;
      it.codes = j.codes;
      it.scales = j.scales;
      it.gs = mx ? nullptr : j.global_scale;
      it.partials = part;
      it.P = qparams(&j.cfg, j.cols);
      items[nitems++] = it;
      if (nitems == kBatchChunk) {
        const int rc = hip_status(fp4lib::launch_quantize_batch(items, nitems, st));
        if (rc != FP4_OK) return rc;
        nitems = 0;
      }
      continue;
    }
    const int rc = mx ? quantize_mx(&j.cfg, j.x, j.xdt, j.rows, j.cols, j.ldx, j.codes, j.scales, st)
                      : quantize_nv_passes(&j.cfg, j.x, j.xdt, j.rows, j.cols, j.ldx, j.codes,
                                           j.scales, j.global_scale, part, st);
    if (rc != FP4_OK) return rc;
  }
  return hip_status(fp4lib::launch_quantize_batch(items, nitems, st));
}

int fp4_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes == 0) return FP4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 7u) != 0 || (ws_bytes & 3u) != 0) return FP4_ERR_ALIGNMENT;
  return hip_status(fp4lib::launch_zero_words(static_cast<uint32_t*>(ws), (int64_t)(ws_bytes / 4),
                                              static_cast<hipStream_t>(stream)));
}

int fp4_quantize_one_pass_fits(const fp4_qconfig* cfg, int32_t xdt, int64_t rows, int64_t cols,
                               int64_t ldx) {
  if (check_cfg(cfg, rows, cols) != FP4_OK || fp4k::fmt_mx(cfg->fmt) || ldx < cols) return 0;
  return fp4lib::quantize_nv_one_pass_tpw(xdt, cfg->block_rows, rows, cols, ldx, kNvExchangeSlots) != 0;
}

int fp4_global_scale(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows,
                     int64_t cols, int64_t ldx, float* global_scale, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_cfg(cfg, rows, cols);
  if (rc != FP4_OK) return rc;
  if (fp4k::fmt_mx(cfg->fmt)) return FP4_ERR_INVALID_ARG;
  rc = check_ld(x, xdt, rows, cols, ldx);
  if (rc != FP4_OK) return rc;
  if (!global_scale) return FP4_ERR_INVALID_ARG;
  if (!ws || ws_bytes < fp4_workspace_bytes(cfg, rows, cols)) return FP4_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return FP4_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0 || cols == 0)
    return hip_status(fp4lib::launch_amax_final(cfg->fmt, nullptr, 0, global_scale, st));
  float* partials = static_cast<float*>(ws);
  const int npart = fp4lib::amax_partials(rows, cols, cfg->rotate != 0, xdt);
  hipError_t e = fp4lib::launch_amax_nv(x, xdt, cfg->rotate != 0, qparams(cfg, cols).signs[0], rows,
                                        cols, ldx, partials, npart, st);
  if (e != hipSuccess) return FP4_ERR_HIP;
  return hip_status(fp4lib::launch_amax_final(cfg->fmt, partials, npart, global_scale, st));
}

int fp4_dequantize(const fp4_qconfig* cfg, const uint8_t* codes, const uint8_t* scales,
                   const float* global_scale, int64_t rows, int64_t cols, void* y, int32_t ydt,
                   int64_t ldy, int32_t inverse_rotate, void* stream) {
  int rc = check_cfg(cfg, rows, cols);
  if (rc != FP4_OK) return rc;
  rc = check_ld(y, ydt, rows, cols, ldy);
  if (rc != FP4_OK) return rc;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales) return FP4_ERR_INVALID_ARG;
  if (!aligned16(codes)) return FP4_ERR_ALIGNMENT;
  if (!fp4k::fmt_mx(cfg->fmt) && !global_scale) return FP4_ERR_INVALID_ARG;
  const int rot = inverse_rotate != 0 ? rot_blocks(cfg) : 0;
  return hip_status(fp4lib::launch_dequantize(cfg->fmt, rot, gemm_layout(cfg) ? 1 : 0, codes, scales,
                                              global_scale, rows, cols, y, ydt, ldy,
                                              qparams(cfg, cols), static_cast<hipStream_t>(stream)));
}

size_t fp4_error_workspace_bytes(const fp4_qconfig* cfg, int64_t rows, int64_t cols) {
  if (check_cfg(cfg, rows, cols) != FP4_OK) return 0;
  return (size_t)fp4lib::error_partials(rows, cols, cfg->fmt) * 4 * sizeof(double);
}

int fp4_error_sums(const fp4_qconfig* cfg, const void* x, int32_t xdt, int64_t rows, int64_t cols,
                   int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                   const float* global_scale, double* sums, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check_cfg(cfg, rows, cols);
  if (rc != FP4_OK) return rc;
  rc = check_ld(x, xdt, rows, cols, ldx);
  if (rc != FP4_OK) return rc;
  if (!sums) return FP4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sums) & 7u) != 0) return FP4_ERR_ALIGNMENT;
  if (!ws || ws_bytes < fp4_error_workspace_bytes(cfg, rows, cols)) return FP4_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 7u) != 0) return FP4_ERR_ALIGNMENT;
  if (rows > 0 && cols > 0) {
    if (!codes || !scales) return FP4_ERR_INVALID_ARG;
    if (!aligned16(codes)) return FP4_ERR_ALIGNMENT;
    if (!fp4k::fmt_mx(cfg->fmt) && !global_scale) return FP4_ERR_INVALID_ARG;
  }
  return hip_status(fp4lib::launch_error_sums(cfg->fmt, rot_blocks(cfg), gemm_layout(cfg) ? 1 : 0,
                                              x, xdt, ldx, codes, scales, global_scale, rows, cols,
                                              sums, static_cast<double*>(ws), qparams(cfg, cols),
                                              static_cast<hipStream_t>(stream)));
}

int fp4_scales_to_gemm_layout(const fp4_qconfig* cfg, const uint8_t* rowmajor, int64_t rows,
                              int64_t cols, uint8_t* gemm_scales, void* stream) {
  int rc = check_cfg(cfg, rows, cols);
  if (rc != FP4_OK) return rc;
  if (!fp4k::fmt_mx(cfg->fmt)) return FP4_ERR_UNSUPPORTED;  // NV formats: the layouts coincide
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!rowmajor || !gemm_scales) return FP4_ERR_INVALID_ARG;
  return hip_status(fp4lib::launch_scales_to_gemm(rowmajor, rows, cols, gemm_scales,
                                                  static_cast<hipStream_t>(stream)));
}

// fmt of the GEMM calls: the format, possibly with FP4_GEMM_B_TILED.  Returns
// the format, -1 for unknown bits; *bt the B layout flag.
int32_t gemm_fmt(int32_t fmt, int* bt) {
  *bt = (fmt & FP4_GEMM_B_TILED) != 0 ? 1 : 0;
  const int32_t f = fmt & ~(int32_t)FP4_GEMM_B_TILED;
  return (f < FP4_FMT_MXFP4 || f > FP4_FMT_NVINT4) ? -1 : f;
}

size_t fp4_gemm_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K) {
  int bt;
  fmt = gemm_fmt(fmt, &bt);
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return 0;
  if (fmt == FP4_FMT_MXFP4) return fp4lib::gemm_mx_workspace(M, N, K);
  if (fmt == FP4_FMT_NVFP4 || fmt == FP4_FMT_MXINT4 || fmt == FP4_FMT_NVINT4)
    return fp4lib::gemm_nv_workspace(fmt, M, N, K);
  return 0;
}

int fp4_gemm(int32_t fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
             const uint8_t* a_scales, const float* a_gs, const uint8_t* b_codes,
             const uint8_t* b_scales, const float* b_gs, void* y, int32_t ydt, int64_t ldy,
             void* ws, size_t ws_bytes, void* stream) {
  int bt;
  fmt = gemm_fmt(fmt, &bt);
  if (fmt < 0) return FP4_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID_ARG;
  if (bt && N % 128 != 0) return FP4_ERR_INVALID_ARG;
  if (K % 128 != 0) return FP4_ERR_UNSUPPORTED;
  if (fp4k::fmt_int(fmt) && K % 256 != 0) return FP4_ERR_UNSUPPORTED;
  if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
    return FP4_ERR_UNSUPPORTED;
  if (dtype_bytes(ydt) == 0) return FP4_ERR_INVALID_ARG;
  if (ldy < N) return FP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP4_OK;
  if (!y) return FP4_ERR_INVALID_ARG;
  if (K > 0) {
    if (!a_codes || !a_scales || !b_codes || !b_scales) return FP4_ERR_INVALID_ARG;
    if (!aligned16(a_codes) || !aligned16(b_codes)) return FP4_ERR_ALIGNMENT;
    if (!aligned16(a_scales) || !aligned16(b_scales)) return FP4_ERR_ALIGNMENT;
  }
  if (ws && !aligned16(ws)) return FP4_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fmt == FP4_FMT_MXFP4)
    return hip_status(fp4lib::launch_gemm_mx(M, N, K, a_codes, a_scales, b_codes, b_scales, bt, y,
                                             ydt, ldy, ws, ws_bytes, st));
  if (fmt == FP4_FMT_MXINT4)
    return hip_status(fp4lib::launch_gemm_int4(fmt, M, N, K, a_codes, a_scales, nullptr, b_codes,
                                               b_scales, nullptr, bt, y, ydt, ldy, ws, ws_bytes, st));
  if (!a_gs || !b_gs) return FP4_ERR_INVALID_ARG;
  if (fmt == FP4_FMT_NVINT4)
    return hip_status(fp4lib::launch_gemm_int4(fmt, M, N, K, a_codes, a_scales, a_gs, b_codes,
                                               b_scales, b_gs, bt, y, ydt, ldy, ws, ws_bytes, st));
  return hip_status(fp4lib::launch_gemm_nv(M, N, K, a_codes, a_scales, a_gs, b_codes, b_scales,
                                           b_gs, bt, y, ydt, ldy, ws, ws_bytes, st));
}

size_t fp4_gemm_w4a16_workspace_bytes(int32_t fmt, int64_t M, int64_t N, int64_t K) {
  int bt;
  fmt = gemm_fmt(fmt, &bt);
  if (fmt < 0) return 0;
  if (M < 0 || N < 0 || K < 0 || K % 256 != 0) return 0;
  return fp4lib::gemm_w4a16_workspace(M, N, K);
}

int fp4_gemm_w4a16(int32_t fmt, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                   const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gs, void* y,
                   int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int bt;
  fmt = gemm_fmt(fmt, &bt);
  if (fmt < 0) return FP4_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID_ARG;
  if (bt && N % 128 != 0) return FP4_ERR_INVALID_ARG;
  if (K % 256 != 0) return FP4_ERR_UNSUPPORTED;
  if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
    return FP4_ERR_UNSUPPORTED;
  if (dtype_bytes(ydt) == 0) return FP4_ERR_INVALID_ARG;
  if (ldy < N) return FP4_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FP4_OK;
  if (!y) return FP4_ERR_INVALID_ARG;
  if (K > 0) {
    if (!a || !b_codes || !b_scales) return FP4_ERR_INVALID_ARG;
    if (lda < K) return FP4_ERR_INVALID_ARG;
    if (!aligned16(a) || (M > 1 && (lda * 2) % 16 != 0)) return FP4_ERR_ALIGNMENT;
    if (!aligned16(b_codes) || !aligned16(b_scales)) return FP4_ERR_ALIGNMENT;
    if (!fp4k::fmt_mx(fmt) && !b_gs) return FP4_ERR_INVALID_ARG;
  }
  if (ws && !aligned16(ws)) return FP4_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(fp4lib::launch_gemm_w4a16(fmt, M, N, K, a, lda, b_codes, b_scales, b_gs, bt,
                                              y, ydt, ldy, ws, ws_bytes, st));
}

}  // extern "C"
