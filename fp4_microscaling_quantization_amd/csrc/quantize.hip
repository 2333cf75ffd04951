// quantize.hip -- block-wise MXFP4 / NVFP4 quantization kernels for gfx950.
//
// One thread owns one quantization block (32 elements for MXFP4, 16 for
// NVFP4): it loads the block with 16-byte vector loads, optionally applies the
// block Hadamard in registers, reduces the block amax, derives the scale,
// encodes the elements with the hardware FP4 conversion and stores the packed
// codes with one 16-byte (MXFP4) or 8-byte (NVFP4) store, so that consecutive
// lanes write consecutive bytes.
//
// Method (pages cited by title):
//  * MXFP4: scale exponent floor(log2(amax)) - 2, E8M0 code clamped to
//    [0, 254]; elements rounded to nearest-even on the E2M1 grid with
//    saturation ("NVFP4 vs MXFP4: 4-Bit Floating Point for LLM Training and
//    Inference (2026)", "A worked example, by hand" and the emulation section;
//    "Bridging the Gap Between Promise and Performance for Microscaling FP4
//    Quantization", format definitions).
//  * NVFP4: ts = amax_tensor / 2688; block code = E4M3(RNE, <= 448) of
//    (amax / 6) / ts; elements use q = fl32(x / (e4m3 * ts)) (NVFP4 vs MXFP4,
//    Figure 2 and the emulation's nvfp4).
//  * Rotation: block Hadamard of the block size, Sylvester order, / sqrt(n)
//    ("Bridging the Gap ...": group-level rotations Q(X H_k); "Portable FP4
//    Quantization for Heterogeneous Accelerators", section 2.3: the block
//    transform fused as an activation butterfly).
#include "fp4_device.h"
#include "launch.h"

using namespace fp4k;

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- loaders
// Load the G elements of block (r, kb) as fp32.
template <int G, int XDT>
__device__ __forceinline__ void load_block_f32(const void* __restrict__ x, int64_t ldx, int64_t r,
                                               int64_t kb, float* v) {
  if constexpr (XDT == FP4_DT_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + r * ldx +
                                                    kb * G);
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
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + r * ldx + kb * G);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      f32x4 w = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = w[j];
    }
  }
}

__device__ __forceinline__ uint32_t mx_code_from_amax(float amax) {
  // floor(log2(amax)) = exponent field - 127 for normal amax; subnormal and
  // zero amax clamp to the smallest scale (code 0).
  int ef = (int)((as_u(amax) >> 23) & 0xFFu);
  return (uint32_t)max(ef - 2, 0);
}

__device__ __forceinline__ void store_mx_scale(uint8_t* __restrict__ scales, int64_t r, int64_t kb,
                                               int64_t nb, int64_t kchunks, bool gemm_layout,
                                               uint32_t code) {
  int64_t off = gemm_layout ? mx_gemm_scale_offset(r, kb, kchunks) : r * nb + kb;
  scales[off] = (uint8_t)code;
}

// ------------------------------------------------------------------ MXFP4
template <int XDT, bool ROT>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(
    const void* __restrict__ x, int64_t ldx, uint32_t rows, uint32_t nb,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t kchunks, int gemm_layout) {
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    u32x4 out[1];
    uint32_t code;
    if constexpr (XDT == FP4_DT_BF16 && !ROT) {
      // Raw bf16 words: |x| compares as an unsigned 15-bit integer.
      const u32x4* p =
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + (int64_t)r * ldx +
                                         (int64_t)kb * 32);
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 t = p[i];
        w[4 * i] = t[0];
        w[4 * i + 1] = t[1];
        w[4 * i + 2] = t[2];
        w[4 * i + 3] = t[3];
      }
      u16x2 m = {0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
      uint32_t amax_bits = (uint32_t)max(m[0], m[1]);
      int ef = (int)((amax_bits >> 7) & 0xFFu);
      code = (uint32_t)max(ef - 2, 0);
      const float sc = e8m0_as_cvt_scale(code);
      // each enc8 call encodes 8 elements (4 input dwords) into one dword
      out[0][0] = enc8_bf16(&w[0], sc);
      out[0][1] = enc8_bf16(&w[4], sc);
      out[0][2] = enc8_bf16(&w[8], sc);
      out[0][3] = enc8_bf16(&w[12], sc);
    } else {
      float v[32];
      load_block_f32<32, XDT>(x, ldx, r, kb, v);
      if constexpr (ROT) {
        fwht<32>(v);
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = div_sqrt32(v[i]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      code = mx_code_from_amax(amax);
      const float sc = e8m0_as_cvt_scale(code);
      out[0][0] = enc8_f32(&v[0], sc);
      out[0][1] = enc8_f32(&v[8], sc);
      out[0][2] = enc8_f32(&v[16], sc);
      out[0][3] = enc8_f32(&v[24], sc);
    }
    *reinterpret_cast<u32x4*>(codes + (int64_t)r * (nb * 16) + (int64_t)kb * 16) = out[0];
    store_mx_scale(scales, r, kb, nb, kchunks, gemm_layout != 0, code);
  }
}

// ------------------------------------------------------------------ NVFP4
// Per-block scale code and scale value s = e4m3 * ts (fp32).
__device__ __forceinline__ uint32_t nv_block_scale(float amax, float ts, float inv_ts,
                                                   bool ts_exact_path, float* s_out) {
  const float inv6 = 0x1.555556p-3f;  // fl32(1/6)
  float h = (amax < 0x1p-100f) ? amax / 6.0f : div_rn(amax, 6.0f, inv6);
  float t = (ts_exact_path || h < 0x1p-100f) ? h / ts : div_rn(h, ts, inv_ts);
  uint32_t c = e4m3_rne_sat(t);
  *s_out = e4m3_value(c) * ts;
  return c;
}

template <int XDT, bool ROT>
__global__ __launch_bounds__(kThreads) void quant_nv_kernel(
    const void* __restrict__ x, int64_t ldx, uint32_t rows, uint32_t nb,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ gs) {
  const float ts = *gs;
  const bool live = ts > 0.0f;
  const bool ts_small = ts < 0x1p-100f;
  const float inv_ts = live ? 1.0f / ts : 0.0f;
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    float v[16];
    load_block_f32<16, XDT>(x, ldx, r, kb, v);
    if constexpr (ROT) {
      fwht<16>(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] *= 0.25f;  // 1/sqrt(16), exact
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t code = 0;
    float s = 0.0f;
    if (live) code = nv_block_scale(amax, ts, inv_ts, ts_small, &s);
    u32x2 out = {0u, 0u};
    if (s != 0.0f) {
      const float one = 1.0f;  // scale operand 2^0: the quotient is already exact
      if (s >= 0x1p-100f) {
        const float rs = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __builtin_copysignf(div_rn(v[i], s, rs), v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = v[i] / s;
      }
      out[0] = enc8_f32(&v[0], one);
      out[1] = enc8_f32(&v[8], one);
    }
    *reinterpret_cast<u32x2*>(codes + (int64_t)r * (nb * 8) + (int64_t)kb * 8) = out;
    scales[(int64_t)r * nb + kb] = (uint8_t)code;
  }
}

// Global amax of the (optionally rotated) tensor, then ts = amax / 2688 written
// to gs_out by the last workgroup to finish, which also returns ws[0..1] to 0.
template <int XDT, bool ROT>
__global__ __launch_bounds__(kThreads) void amax_nv_kernel(const void* __restrict__ x, int64_t ldx,
                                                           uint32_t rows, uint32_t nb,
                                                           uint32_t* __restrict__ ws,
                                                           float* __restrict__ gs_out) {
  float m = 0.0f;
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    float v[16];
    load_block_f32<16, XDT>(x, ldx, r, kb, v);
    if constexpr (ROT) fwht<16>(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  if constexpr (ROT) m *= 0.25f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) mm = fmaxf(mm, red[i]);
    atomicMax(&ws[0], as_u(mm));
    __threadfence();
    uint32_t ticket = atomicAdd(&ws[1], 1u);
    if (ticket == gridDim.x - 1) {
      __threadfence();
      uint32_t g = atomicExch(&ws[0], 0u);
      atomicExch(&ws[1], 0u);
      *gs_out = as_f(g) / 2688.0f;
    }
  }
}

__global__ void set_scalar_kernel(float* p, float v) { *p = v; }

// Row-major [rows, nb] MXFP4 scales -> GEMM layout (padding filled with 127).
__global__ __launch_bounds__(kThreads) void scales_to_gemm_kernel(const uint8_t* __restrict__ src,
                                                                  uint32_t rows, uint32_t nb,
                                                                  uint32_t kchunks,
                                                                  uint8_t* __restrict__ dst,
                                                                  uint32_t total) {
  for (uint32_t p = blockIdx.x * kThreads + threadIdx.x; p < total; p += gridDim.x * kThreads) {
    uint32_t tile = p >> 8, within = p & 255u;
    uint32_t dw = within >> 2, j = within & 3u;
    uint32_t h = dw >> 5, rr = dw & 31u;
    uint32_t rt = tile / kchunks, kc = tile - rt * kchunks;
    uint32_t r = rt * 32 + rr, kb = kc * 8 + 2 * j + h;
    dst[p] = (r < rows && kb < nb) ? src[(int64_t)r * nb + kb] : (uint8_t)127;
  }
}

int grid_for(int64_t total) {
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

namespace fp4lib {

hipError_t launch_quantize_mx(const void* x, int xdt, int rotate, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* codes, uint8_t* scales, int gemm_layout,
                              hipStream_t st) {
  const uint32_t nb = (uint32_t)(cols / 32);
  const int64_t total = rows * (int64_t)nb;
  const int64_t kchunks = mx_gemm_kchunks(cols);
  const int grid = grid_for(total);
#define FP4_QMX(XDT, ROT)                                                                   \
  quant_mx_kernel<XDT, ROT><<<grid, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, nb, codes, scales, \
                                                       kchunks, gemm_layout)
  if (xdt == FP4_DT_BF16) {
    if (rotate) FP4_QMX(FP4_DT_BF16, true); else FP4_QMX(FP4_DT_BF16, false);
  } else {
    if (rotate) FP4_QMX(FP4_DT_F32, true); else FP4_QMX(FP4_DT_F32, false);
  }
#undef FP4_QMX
  return hipGetLastError();
}

hipError_t launch_amax_nv(const void* x, int xdt, int rotate, int64_t rows, int64_t cols,
                          int64_t ldx, uint32_t* ws, float* gs_out, hipStream_t st) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const int64_t total = rows * (int64_t)nb;
  if (total == 0) {
    set_scalar_kernel<<<1, 1, 0, st>>>(gs_out, 0.0f);
    return hipGetLastError();
  }
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 2048) g = 2048;
  const int grid = (int)g;
#define FP4_AMX(XDT, ROT) \
  amax_nv_kernel<XDT, ROT><<<grid, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, nb, ws, gs_out)
  if (xdt == FP4_DT_BF16) {
    if (rotate) FP4_AMX(FP4_DT_BF16, true); else FP4_AMX(FP4_DT_BF16, false);
  } else {
    if (rotate) FP4_AMX(FP4_DT_F32, true); else FP4_AMX(FP4_DT_F32, false);
  }
#undef FP4_AMX
  return hipGetLastError();
}

hipError_t launch_quantize_nv(const void* x, int xdt, int rotate, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* codes, uint8_t* scales, const float* gs,
                              hipStream_t st) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const int64_t total = rows * (int64_t)nb;
  const int grid = grid_for(total);
#define FP4_QNV(XDT, ROT) \
  quant_nv_kernel<XDT, ROT><<<grid, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, nb, codes, scales, gs)
  if (xdt == FP4_DT_BF16) {
    if (rotate) FP4_QNV(FP4_DT_BF16, true); else FP4_QNV(FP4_DT_BF16, false);
  } else {
    if (rotate) FP4_QNV(FP4_DT_F32, true); else FP4_QNV(FP4_DT_F32, false);
  }
#undef FP4_QNV
  return hipGetLastError();
}

hipError_t launch_scales_to_gemm(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                                 hipStream_t st) {
  const uint32_t nb = (uint32_t)(cols / 32);
  const int64_t kchunks = mx_gemm_kchunks(cols);
  const int64_t total = ((rows + 31) / 32) * kchunks * 256;
  if (total == 0) return hipSuccess;
  scales_to_gemm_kernel<<<grid_for(total), kThreads, 0, st>>>(src, (uint32_t)rows, nb,
                                                              (uint32_t)kchunks, dst,
                                                              (uint32_t)total);
  return hipGetLastError();
}

}  // namespace fp4lib
