// launch.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4.h"
#include "fp4_device.h"

namespace fp4lib {

hipError_t launch_quantize_mx(int fmt, const void* x, int xdt, int rot_blocks, int rule,
                              int rounding, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                              uint8_t* scales, int gemm_layout, const fp4k::QParams& P,
                              hipStream_t st);
int amax_partials(int64_t rows, int64_t cols, int rotate, int xdt);
hipError_t launch_amax_nv(const void* x, int xdt, int rotate, uint32_t sign_mask, int64_t rows,
                          int64_t cols, int64_t ldx, float* partials, int npart, hipStream_t st);
hipError_t launch_amax_final(int fmt, const float* partials, int npart, float* gs, hipStream_t st);
hipError_t launch_quantize_nv(int fmt, const void* x, int xdt, int rotate, int rule, int rounding,
                              int block_rows, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* gs, const float* partials,
                              int npart, const fp4k::QParams& P, hipStream_t st);
// Single pass (tensor maximum and encoding in one launch); hipErrorNotSupported
// (nothing launched) when the shape or configuration does not fit it.
// xchg: the exchange region (zero before its first use), max_grid slots.
// quantize_nv_one_pass_tpw: wave tiles per wave the single pass would use
// (4 or 8), 0 when it does not apply.
int quantize_nv_one_pass_tpw(int xdt, int block_rows, int64_t rows, int64_t cols, int64_t ldx,
                             int max_grid);
hipError_t launch_quantize_nv_one_pass(int fmt, const void* x, int xdt, int rotate, int rule,
                                       int rounding, int block_rows, int64_t rows, int64_t cols,
                                       int64_t ldx, uint8_t* codes, uint8_t* scales, float* gs,
                                       uint32_t* xchg, int max_grid, const fp4k::QParams& P,
                                       hipStream_t st);
// One quantization of a grouped launch: bf16 input, absmax block scales,
// nearest rounding, one-row blocks, no rotation or the block-sized one
// (rotate != 0), rows > 0 and cols > 0.  partials: nullptr for the MX
// formats and for NVFP4 / NVINT4 with the tensor scale given in *gs;
// otherwise 2048 bytes for the maxima of the tensor-scale pass (the first
// launch writes them, the second launch encodes from them and stores *gs).
struct BatchItem {
  int fmt, rotate, gemm_layout;
  const void* x;
  int64_t rows, cols, ldx;
  uint8_t* codes;
  uint8_t* scales;
  float* gs;
  float* partials;
  fp4k::QParams P;
};
// All items in at most two launches of one kernel (more when there are more
// than 16 per launch).
hipError_t launch_quantize_batch(const BatchItem* items, int n, hipStream_t st);
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st);
hipError_t launch_scales_to_gemm(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                                 hipStream_t st);

hipError_t launch_dequantize(int fmt, int rot_blocks, int gemm_layout, const uint8_t* codes,
                             const uint8_t* scales, const float* gs, int64_t rows, int64_t cols,
                             void* y, int ydt, int64_t ldy, const fp4k::QParams& P, hipStream_t st);
int error_partials(int64_t rows, int64_t cols, int fmt);
hipError_t launch_error_sums(int fmt, int rot_blocks, int gemm_layout, const void* x, int xdt,
                             int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                             const float* gs, int64_t rows, int64_t cols, double* sums,
                             double* partials, const fp4k::QParams& P, hipStream_t st);

size_t gemm_mx_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const uint8_t* b, const uint8_t* bs, int bt, void* y, int ydt, int64_t ldy,
                          void* ws, size_t ws_bytes, hipStream_t st);
size_t gemm_nv_workspace(int fmt, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_nv(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                          int bt, void* y, int ydt, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t st);

hipError_t launch_gemm_int4(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                            const uint8_t* as, const float* ags, const uint8_t* b, const uint8_t* bs,
                            const float* bgs, int bt, void* y, int ydt, int64_t ldy, void* ws,
                            size_t ws_bytes, hipStream_t st);

size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w4a16(int fmt, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                             const uint8_t* b, const uint8_t* bs, const float* bgs, int bt, void* y,
                             int ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace fp4lib
