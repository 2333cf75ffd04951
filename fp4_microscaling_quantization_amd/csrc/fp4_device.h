// fp4_device.h -- device-side helpers shared by the gfx950 kernels of this
// library (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4k {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Formats: E8M0 block scales (MX) or E4M3 block scales with an fp32 tensor
// scale (NV); E2M1 or INT4 element.
__host__ __device__ constexpr bool fmt_mx(int f) { return f == 0 || f == 2; }
__host__ __device__ constexpr bool fmt_int(int f) { return f == 2 || f == 3; }
__host__ __device__ constexpr int fmt_block(int f) { return fmt_mx(f) ? 32 : 16; }
// Largest element magnitude: 6 (E2M1) or 7 (INT4).
__host__ __device__ constexpr float fmt_qmax(int f) { return fmt_int(f) ? 7.0f : 6.0f; }

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// bf16 pair (low half = element 0) widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = as_u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- E2M1 encode
// The gfx950 conversion v_cvt_scalef32_pk_fp4_* rounds x / 2^E to the nearest
// E2M1 value with ties to even, saturates at +-6 and keeps the sign of zero,
// where E is taken from the exponent field of the scale operand alone (field 0
// means 2^-127).  Passing the E8M0 code shifted into the exponent field makes
// it divide by exactly the MXFP4 block scale.
__device__ __forceinline__ float e8m0_as_cvt_scale(uint32_t code) { return as_f(code << 23); }

// Eight fp32 values -> one dword of codes (element 0 in the low nibble).
__device__ __forceinline__ uint32_t enc8_f32(const float* v, float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], scale, 3);
  return r;
}

// Eight bf16 values (four packed dwords) -> one dword of codes.
__device__ __forceinline__ uint32_t enc8_bf16(const uint32_t* w, float scale) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w[0]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w[1]), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w[2]), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, as_bf16x2(w[3]), scale, 3);
  return r;
}

// ---------------------------------------------------------------- E2M1 decode
// One byte of codes -> two fp32 values times 2^E (E from the scale's exponent
// field, as above).  Exact.
__device__ __forceinline__ f32x2 dec2_f32(uint32_t byte_src, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte_src, scale, 0);
}

// 2^(code - 127) as an fp32 value (code 0: the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  return code == 0u ? as_f(0x00400000u) : as_f(code << 23);
}

// ---------------------------------------------------------------- INT4
// Nearest integer (ties to even) of q clipped to [-7, 7], as a nibble.
__device__ __forceinline__ uint32_t int4_nibble(float q) {
  const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(q), -7.0f, 7.0f);
  return (uint32_t)(int)r & 15u;
}

// Eight quotients -> one dword of INT4 codes (element 0 in the low nibble).
__device__ __forceinline__ uint32_t int4_pack8(const float* q) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) r |= int4_nibble(q[i]) << (4 * i);
  return r;
}

// INT4 code i of a dword (sign-extended) as fp32.
__device__ __forceinline__ float int4_value(uint32_t w, int i) {
  return (float)((int32_t)(w << (28 - 4 * i)) >> 28);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: tile arithmetic derived from it runs on the scalar unit.
__device__ __forceinline__ uint32_t wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// ------------------------------------------------------------------ E4M3
// Value of a non-negative E4M3 code (0 .. 0x7E).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  if (code < 8u) return (float)code * 0x1p-9f;
  return as_f((((code >> 3) + 120u) << 23) | ((code & 7u) << 20));
}

// Nearest E4M3 code to t >= 0 (ties to even), after clipping t to 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  t = fminf(t, 448.0f);
  if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);
  uint32_t u = as_u(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);
}

// ------------------------------------------------------------ exact quotient
// fl32(a / b) from r = fl32(1 / b) with two FMAs (Markstein's correction: when
// r is the correctly rounded reciprocal and q0 = fl32(a * r) is within one ulp
// of a / b, the remainder a - q0 * b is exact and fl32(q0 + rem * r) is the
// correctly rounded quotient).  Valid for normal a, b and a normal quotient;
// callers route blocks with tiny scales through an IEEE division instead.
__device__ __forceinline__ float div_rn(float a, float b, float r) {
  float q0 = a * r;
  float rem = __builtin_fmaf(-q0, b, a);
  return __builtin_fmaf(rem, r, q0);
}

// -fl32(a / b) for b > 0, zero sign included (a = +0 gives -0, a = -0 gives
// +0), as -rem * r - q0 with one rounding: round-to-nearest-even is
// symmetric, so every non-zero result is the negated quotient above.  E2M1
// is sign-magnitude, so encoding the negated quotient and flipping every
// code's sign bit gives the codes of the quotient itself.
__device__ __forceinline__ float neg_div_rn(float a, float b, float r) {
  float q0 = a * r;
  float rem = __builtin_fmaf(-q0, b, a);
  return __builtin_fmaf(-rem, r, -q0);
}

// --------------------------------------------------------------- Hadamard
// In-place unnormalised Walsh-Hadamard transform (Sylvester order) of N
// registers.
template <int N>
__device__ __forceinline__ void fwht(float* v) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Correctly rounded (up to a ~2^-47 relative band) y = s / sqrt(32) using a
// two-term constant: fl32(s * c_hi + fl32(s * c_lo)).
__device__ __forceinline__ float div_sqrt32(float s) {
  const float c_hi = 0x1.6a09e6p-3f;          // fl32(1/sqrt(32))
  const float c_lo = 0x1.9fcef4p-29f;         // fl32(1/sqrt(32) - c_hi)
  return __builtin_fmaf(s, c_hi, s * c_lo);
}

// ------------------------------------------------------- quad lane exchange
// DPP quad permutations: lane i of every group of four reads lane i^1 / i^2.
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1(float v) { return as_f(quad_xor1(as_u(v))); }
__device__ __forceinline__ float quad_xor2(float v) { return as_f(quad_xor2(as_u(v))); }

// One butterfly stage of the Walsh-Hadamard transform across lanes: element i
// of lane l pairs with element i of lane l ^ B (B = 1 or 2).  The lower lane
// keeps a + b, the upper one a - b (a = lower lane's value), as the in-register
// stage does for the pair (j, j + h).
template <int B>
__device__ __forceinline__ void fwht_lane_stage(float* v, int lane) {
  const bool up = (lane & B) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = B == 1 ? quad_xor1(v[i]) : quad_xor2(v[i]);
    v[i] = up ? p - v[i] : v[i] + p;
  }
}

// ----------------------------------------------- rotation groups and signs
// Launch parameters beyond the format: the sign diagonal of the rotation
// (bit i of the 128-bit mask: element i of each rotation group negated before
// the transform) and the stochastic-rounding key.
struct QParams {
  uint32_t signs[4];
  uint32_t any_sign;  // nonzero when some sign bit is set
  uint32_t seed0, seed1;
  uint32_t tiled;     // nonzero: codes in the tiled layout (code_offset)
  int64_t cols;       // row length, for the element index of stochastic rounding
};

// Negate element i of the N values when bit i of m is set.
template <int N>
__device__ __forceinline__ void apply_signs(float* v, uint32_t m) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = as_f(as_u(v[i]) ^ (((m >> i) & 1u) << 31));
}

// The sign bits of block kb of a row (blocks of G elements, rotation groups of
// RN blocks): word kb % RN of the mask for G = 32, the low 16 bits for G = 16.
template <int G, int RN>
__device__ __forceinline__ uint32_t block_signs(const QParams& P, uint32_t kb) {
  return P.signs[RN >= 2 ? (kb & (RN - 1)) : 0];
}

// Unnormalised Walsh-Hadamard transform of a rotation group of RN blocks: the
// in-register transform of the lane's block, then log2(RN) butterfly stages
// across the lanes that hold the group's other blocks (consecutive lanes hold
// consecutive blocks, so the partner of block kb for stage d is lane ^ d;
// every lane of a group takes part).  H_(RN G) = H_RN (x) H_G, Sylvester order.
template <int G, int RN>
__device__ __forceinline__ void fwht_group(float* v, uint32_t kb) {
  fwht<G>(v);
  if constexpr (RN >= 2) {
    const bool up = (kb & 1u) != 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float p = quad_xor1(v[i]);
      v[i] = up ? p - v[i] : v[i] + p;
    }
  }
  if constexpr (RN >= 4) {
    const bool up = (kb & 2u) != 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float p = quad_xor2(v[i]);
      v[i] = up ? p - v[i] : v[i] + p;
    }
  }
}

// y = S / sqrt(N) for N = 16 .. 128 (exact for 16 and 64; the two-term
// constant for 32; for 128 that result halved, exactly).
template <int N>
__device__ __forceinline__ float div_sqrt_n(float s) {
  if constexpr (N == 16) return s * 0.25f;
  else if constexpr (N == 32) return div_sqrt32(s);
  else if constexpr (N == 64) return s * 0.125f;
  else return div_sqrt32(s) * 0.5f;
}

// Forward rotation of the lane's block (signs, transform, normalisation).
template <int G, int RN>
__device__ __forceinline__ void rotate_block(float* v, uint32_t kb, const QParams& P) {
  if (P.any_sign) apply_signs<G>(v, block_signs<G, RN>(P, kb));
  fwht_group<G, RN>(v, kb);
#pragma unroll
  for (int i = 0; i < G; ++i) v[i] = div_sqrt_n<G * RN>(v[i]);
}

// Inverse rotation: transform, normalisation, then the signs.
template <int G, int RN>
__device__ __forceinline__ void unrotate_block(float* v, uint32_t kb, const QParams& P) {
  fwht_group<G, RN>(v, kb);
#pragma unroll
  for (int i = 0; i < G; ++i) v[i] = div_sqrt_n<G * RN>(v[i]);
  if (P.any_sign) apply_signs<G>(v, block_signs<G, RN>(P, kb));
}

// ------------------------------------------------------ stochastic rounding
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32 x 32 -> 64-bit products and xors with the key; the key advances by two
// Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t* c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Random words of elements base .. base + N - 1 of the tensor (base a multiple
// of 4): word e % 4 of Philox4x32-10(counter = (e / 4, high half, 0, 0),
// key = seed).
template <int N>
__device__ __forceinline__ void sr_words(uint64_t base, const QParams& P, uint32_t* w) {
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const uint64_t g = (base >> 2) + (uint64_t)j;
    uint32_t c[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
    philox4x32_10(c, P.seed0, P.seed1);
    w[4 * j] = c[0];
    w[4 * j + 1] = c[1];
    w[4 * j + 2] = c[2];
    w[4 * j + 3] = c[3];
  }
}

// Stochastic rounding of quotient q onto the E2M1 grid with the random word w:
// a = min(|q|, 6) between neighbours lo <= a < lo + step rounds up when
// u = (w >> 8) 2^-24 < (a - lo) / step.  Every step is exact (power-of-two
// spacings), so the decision equals the exact comparison.  Returns the grid
// value with the sign of q.
__device__ __forceinline__ float sr_e2m1(float q, uint32_t w) {
  const float a = fminf(fabsf(q), 6.0f);
  const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
  const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
  const float lo = floorf(a * inv) * step;
  const float p = (a - lo) * inv;
  const float u = (float)(w >> 8) * 0x1p-24f;
  return copysignf(u < p ? lo + step : lo, q);
}

// Eight quotients rounded stochastically, as one dword of E2M1 codes (the
// hardware conversion of exact grid values, scale 2^0).
__device__ __forceinline__ uint32_t enc8_sr(const float* q, const uint32_t* w) {
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = sr_e2m1(q[i], w[i]);
  return enc8_f32(g, 1.0f);
}

// ------------------------------------------------------------- scale layout
// MXFP4 GEMM scale layout: one 256-byte tile per (32 rows) x (8 blocks of 32 =
// 256 K).  Within a tile, dword (kb % 2) * 32 + (r % 32) holds the scales of
// row r for blocks kb with the same parity, one byte per 64-K MFMA step: byte
// (kb % 8) / 2.  A lane l of the 32x32x64 scaled MFMA reads dword l.
__host__ __device__ __forceinline__ int64_t mx_gemm_scale_offset(int64_t r, int64_t kb,
                                                                int64_t kchunks) {
  return ((r >> 5) * kchunks + (kb >> 3)) * 256 + (((kb & 1) * 32 + (r & 31)) * 4) +
         ((kb & 7) >> 1);
}

__host__ __device__ __forceinline__ int64_t mx_gemm_kchunks(int64_t cols) {
  return (cols + 255) / 256;
}

// Byte b of row r of a packed-code matrix with row_bytes bytes per row.
// Row-major: r * row_bytes + b.  Tiled (rows and row_bytes multiples of 128
// and 64): 8 KB tiles of 128 rows x 64 bytes (128 elements), row-major inside
// the tile; the tiles of one 128-row panel follow each other along the row,
// and the panels follow each other.  A GEMM stage of 128 rows x 128 K of the
// weights is then one contiguous 8 KB block.
__host__ __device__ __forceinline__ int64_t code_offset(int64_t r, int64_t b, int64_t row_bytes,
                                                        bool tiled) {
  return tiled ? ((((r >> 7) * (row_bytes >> 6) + (b >> 6)) << 13) + ((r & 127) << 6) + (b & 63))
               : r * row_bytes + b;
}

}  // namespace fp4k
