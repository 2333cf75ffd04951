// dequant.hip -- dequantization and error-sum kernels for gfx950.
//
// Dequantization multiplies each E2M1 element by its block scale: E8M0 for
// MXFP4, E4M3 times the fp32 tensor scale for NVFP4 ("NVFP4 vs MXFP4: 4-Bit
// Floating Point for LLM Training and Inference (2026)", Figure 1; "Microscaling
// Formats in Production LLM Inference", format specifications).  With
// inverse rotation the block Hadamard is applied again (it is its own inverse),
// returning to the original domain ("Portable FP4 Quantization for
// Heterogeneous Accelerators", section 2.3, eq. (2)).
//
// The error sums are NMSE's and cosine similarity's ingredients (same page,
// section 3.2), accumulated in double with a fixed reduction order.
#include "fp4_device.h"
#include "launch.h"

using namespace fp4k;

namespace {

constexpr int kThreads = 256;

// Decode block (r, kb) into fp32 values (original domain if INV).
//   MXFP4: e2m1 * 2^e (hardware decode with the E8M0 code as its scale).
//   MXINT4: q * 2^e.  NVFP4 / NVINT4: fl32(fl32(element * e4m3) * ts), the
//   inner product exact.
//   INV != 0: back to the original domain through the inverse of a rotation
//   group of INV blocks (the lanes of a group are consecutive blocks).
template <int FMT, int INV>
__device__ __forceinline__ void decode_block(const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ scales, float ts,
                                             uint32_t r, uint32_t kb, uint32_t nb,
                                             int64_t kchunks, bool gemm_layout, float* v,
                                             const QParams& P) {
  constexpr int G = fmt_block(FMT);
  constexpr int NDW = G / 8;
  uint32_t w[NDW];
  if constexpr (fmt_mx(FMT)) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(codes + code_offset(r, (int64_t)kb * 16, (int64_t)nb * 16, P.tiled != 0));
    w[0] = t[0];
    w[1] = t[1];
    w[2] = t[2];
    w[3] = t[3];
    const int64_t off = gemm_layout ? mx_gemm_scale_offset(r, kb, kchunks) : (int64_t)r * nb + kb;
    if constexpr (fmt_int(FMT)) {
      const float p = e8m0_value(scales[off]);
#pragma unroll
      for (int i = 0; i < NDW; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = int4_value(w[i], j) * p;
    } else {
      const float sc = e8m0_as_cvt_scale(scales[off]);
#pragma unroll
      for (int i = 0; i < NDW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 p = dec2_f32(w[i] >> (8 * j), sc);
          v[8 * i + 2 * j] = p[0];
          v[8 * i + 2 * j + 1] = p[1];
        }
    }
  } else {
    const u32x2 t = *reinterpret_cast<const u32x2*>(codes + code_offset(r, (int64_t)kb * 8, (int64_t)nb * 8, P.tiled != 0));
    w[0] = t[0];
    w[1] = t[1];
    const float e4 = e4m3_value(scales[(int64_t)r * nb + kb]);
    if constexpr (fmt_int(FMT)) {
#pragma unroll
      for (int i = 0; i < NDW; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = (int4_value(w[i], j) * e4) * ts;
    } else {
#pragma unroll
      for (int i = 0; i < NDW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 p = dec2_f32(w[i] >> (8 * j), 1.0f);
          v[8 * i + 2 * j] = (p[0] * e4) * ts;
          v[8 * i + 2 * j + 1] = (p[1] * e4) * ts;
        }
    }
  }
  if constexpr (INV != 0) unrotate_block<G, INV>(v, kb, P);
}

template <int FMT, int INV, int YDT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gs, uint32_t rows, uint32_t nb, int64_t kchunks, int gemm_layout,
    void* __restrict__ y, int64_t ldy, QParams P) {
  constexpr int G = fmt_block(FMT);
  const float ts = fmt_mx(FMT) ? 0.0f : *gs;
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    float v[G];
    decode_block<FMT, INV>(codes, scales, ts, r, kb, nb, kchunks, gemm_layout != 0, v, P);
    if constexpr (YDT == FP4_DT_F32) {
      f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(y) + (int64_t)r * ldy + (int64_t)kb * G);
#pragma unroll
      for (int i = 0; i < G / 4; ++i) p[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    } else {
      u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + (int64_t)r * ldy + (int64_t)kb * G);
#pragma unroll
      for (int i = 0; i < G / 8; ++i) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = f32_to_bf16_rne(v[8 * i + 2 * j]) | (f32_to_bf16_rne(v[8 * i + 2 * j + 1]) << 16);
        p[i] = o;
      }
    }
  }
}

template <int XDT, int G>
__device__ __forceinline__ void load_x(const void* __restrict__ x, int64_t ldx, uint32_t r,
                                       uint32_t kb, float* v) {
  if constexpr (XDT == FP4_DT_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) +
                                                    (int64_t)r * ldx + (int64_t)kb * G);
#pragma unroll
    for (int i = 0; i < G / 8; ++i) {
      u32x4 w = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_lo(w[j]);
        v[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) +
                                                    (int64_t)r * ldx + (int64_t)kb * G);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      f32x4 w = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
    }
  }
}

__device__ __forceinline__ double shfl_xor_d(double v, int off) {
  return __shfl_xor(v, off, 64);
}

// Per-workgroup partial sums [gridDim.x][4] in double.
template <int FMT, int INV, int XDT>
__global__ __launch_bounds__(kThreads) void error_partial_kernel(
    const void* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ gs, uint32_t rows, uint32_t nb,
    int64_t kchunks, int gemm_layout, double* __restrict__ partials, QParams P) {
  constexpr int G = fmt_block(FMT);
  const float ts = fmt_mx(FMT) ? 0.0f : *gs;
  double se = 0.0, sx = 0.0, sxy = 0.0, sy = 0.0;
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    float v[G], xv[G];
    decode_block<FMT, INV>(codes, scales, ts, r, kb, nb, kchunks, gemm_layout != 0, v, P);
    load_x<XDT, G>(x, ldx, r, kb, xv);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      double a = xv[i], h = v[i];
      double d = a - h;
      se = __builtin_fma(d, d, se);
      sx = __builtin_fma(a, a, sx);
      sxy = __builtin_fma(a, h, sxy);
      sy = __builtin_fma(h, h, sy);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    se += shfl_xor_d(se, off);
    sx += shfl_xor_d(sx, off);
    sxy += shfl_xor_d(sxy, off);
    sy += shfl_xor_d(sy, off);
  }
  __shared__ double red[kThreads / 64][4];
  const int wave = (int)wave_index();
  if ((threadIdx.x & 63) == 0) {
    red[wave][0] = se;
    red[wave][1] = sx;
    red[wave][2] = sxy;
    red[wave][3] = sy;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += red[w][threadIdx.x];
    partials[(int64_t)blockIdx.x * 4 + threadIdx.x] = s;
  }
}

// Sum n partial rows of 4 doubles in a fixed order.
__global__ __launch_bounds__(kThreads) void error_final_kernel(const double* __restrict__ partials,
                                                               int n, double* __restrict__ sums) {
  __shared__ double red[kThreads][4];
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < n; i += kThreads) {
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] += partials[(int64_t)i * 4 + c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[threadIdx.x][c] = s[c];
  __syncthreads();
  for (int half = kThreads / 2; half >= 1; half >>= 1) {
    if (threadIdx.x < half) {
#pragma unroll
      for (int c = 0; c < 4; ++c) red[threadIdx.x][c] += red[threadIdx.x + half][c];
    }
    __syncthreads();
  }
  if (threadIdx.x < 4) sums[threadIdx.x] = red[0][threadIdx.x];
}

int grid_for(int64_t total, int cap) {
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

namespace fp4lib {

hipError_t launch_dequantize(int fmt, int rot_blocks, int gemm_layout, const uint8_t* codes,
                             const uint8_t* scales, const float* gs, int64_t rows, int64_t cols,
                             void* y, int ydt, int64_t ldy, const QParams& P, hipStream_t st) {
  const int G = fmt_block(fmt);
  const uint32_t nb = (uint32_t)(cols / G);
  const int64_t total = rows * (int64_t)nb;
  if (total == 0) return hipSuccess;
  const int64_t kchunks = mx_gemm_kchunks(cols);
  const int grid = grid_for(total, 8192);
#define FP4_DQ(F, I, Y)                                                                    \
  dequant_kernel<F, I, Y><<<grid, kThreads, 0, st>>>(codes, scales, gs, (uint32_t)rows, nb, \
                                                     kchunks, gemm_layout, y, ldy, P)
#define FP4_DQ_Y(F, I)                                   \
  do {                                                   \
    if (ydt == FP4_DT_F32) FP4_DQ(F, I, FP4_DT_F32);     \
    else FP4_DQ(F, I, FP4_DT_BF16);                      \
  } while (0)
#define FP4_DQ_R(F)                                                  \
  do {                                                               \
    if (rot_blocks == 0) FP4_DQ_Y(F, 0);                             \
    else if (rot_blocks == 1) FP4_DQ_Y(F, 1);                        \
    else if (fmt_mx(F) && rot_blocks == 2) FP4_DQ_Y(F, 2);           \
    else if (fmt_mx(F) && rot_blocks == 4) FP4_DQ_Y(F, 4);           \
  } while (0)
  if (fmt == FP4_FMT_MXFP4) FP4_DQ_R(FP4_FMT_MXFP4);
  else if (fmt == FP4_FMT_NVFP4) FP4_DQ_R(FP4_FMT_NVFP4);
  else if (fmt == FP4_FMT_MXINT4) FP4_DQ_R(FP4_FMT_MXINT4);
  else FP4_DQ_R(FP4_FMT_NVINT4);
#undef FP4_DQ_R
#undef FP4_DQ_Y
#undef FP4_DQ
  return hipGetLastError();
}

int error_partials(int64_t rows, int64_t cols, int fmt) {
  const int G = fmt_block(fmt);
  return grid_for(rows * (cols / G), 1024);
}

hipError_t launch_error_sums(int fmt, int rot_blocks, int gemm_layout, const void* x, int xdt,
                             int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                             const float* gs, int64_t rows, int64_t cols, double* sums,
                             double* partials, const QParams& P, hipStream_t st) {
  const int G = fmt_block(fmt);
  const uint32_t nb = (uint32_t)(cols / G);
  const int64_t kchunks = mx_gemm_kchunks(cols);
  const int grid = error_partials(rows, cols, fmt);
  if (rows * (int64_t)nb == 0) {
    error_final_kernel<<<1, kThreads, 0, st>>>(partials, 0, sums);
    return hipGetLastError();
  }
#define FP4_ER(F, I, X)                                                                        \
  error_partial_kernel<F, I, X><<<grid, kThreads, 0, st>>>(x, ldx, codes, scales, gs,           \
                                                           (uint32_t)rows, nb, kchunks,         \
                                                           gemm_layout, partials, P)
#define FP4_ER_X(F, I)                                   \
  do {                                                   \
    if (xdt == FP4_DT_F32) FP4_ER(F, I, FP4_DT_F32);     \
    else FP4_ER(F, I, FP4_DT_BF16);                      \
  } while (0)
#define FP4_ER_R(F)                                                  \
  do {                                                               \
    if (rot_blocks == 0) FP4_ER_X(F, 0);                             \
    else if (rot_blocks == 1) FP4_ER_X(F, 1);                        \
    else if (fmt_mx(F) && rot_blocks == 2) FP4_ER_X(F, 2);           \
    else if (fmt_mx(F) && rot_blocks == 4) FP4_ER_X(F, 4);           \
  } while (0)
  if (fmt == FP4_FMT_MXFP4) FP4_ER_R(FP4_FMT_MXFP4);
  else if (fmt == FP4_FMT_NVFP4) FP4_ER_R(FP4_FMT_NVFP4);
  else if (fmt == FP4_FMT_MXINT4) FP4_ER_R(FP4_FMT_MXINT4);
  else FP4_ER_R(FP4_FMT_NVINT4);
#undef FP4_ER_R
#undef FP4_ER_X
#undef FP4_ER
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  error_final_kernel<<<1, kThreads, 0, st>>>(partials, grid, sums);
  return hipGetLastError();
}

}  // namespace fp4lib
