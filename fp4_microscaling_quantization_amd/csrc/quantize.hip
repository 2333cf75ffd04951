// quantize.hip -- block-wise MXFP4 / NVFP4 quantization kernels for gfx950.
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
//
// Work decomposition.  Every quantization block is computed by one thread
// (butterfly, amax, scale and encode all in registers).  In the tiled kernel a
// wave owns 64 consecutive blocks of one row: it loads them with fully
// coalesced 16-byte loads (1 KB per instruction), transposes them through a
// padded LDS buffer so that each lane holds its own block, and stores the
// packed codes with one 16-byte (MXFP4) or 8-byte (NVFP4) store per lane, so
// the wave writes a contiguous range.  Shapes whose rows are not a multiple of
// 64 blocks use the direct kernel (each thread loads its own block).
//
// NVFP4 with a computed tensor scale runs two launches: the amax pass writes
// one partial maximum per workgroup (no atomics), and the quantize pass
// reduces those partials in its prologue.
#include "fp4_device.h"
#include "launch.h"
#include <atomic>

using namespace fp4k;

namespace {

constexpr int kThreads = 256;
constexpr int kAmaxGrid = 512;  // partial maxima written by the amax pass

// ------------------------------------------------------- per-block compute
// Block-scale rules: FP4_SCALE_ABSMAX (the block maximum sets the scale),
// FP4_SCALE_MSE (the candidate code with the smallest block squared error:
// MXFP4 c0, c0 + 1; NVFP4 c0 - 2 .. c0 + 6), FP4_SCALE_FOUR_OVER_SIX (NVFP4:
// the block maximum onto 6 or onto 4, the smaller error) -- "Bridging the Gap
// ...", MR-GPTQ's MSE-optimised scales; "NVFP4 vs MXFP4 ...", the E2M1 grid
// section and Four Over Six.  The error is summed in fp32 in element order with
// one fma per element: d = fl32(y - y^), acc = fma(d, d, acc); a candidate
// replaces the best only with a strictly smaller sum, so ties keep the earlier
// one (the absmax code first).

// Eight codes (one dword) -> their E2M1 grid values (exact, zero sign kept).
__device__ __forceinline__ void decode8(uint32_t w, float* m) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  m[0] = a[0]; m[1] = a[1]; m[2] = b[0]; m[3] = b[1];
  m[4] = c[0]; m[5] = c[1]; m[6] = d[0]; m[7] = d[1];
}

// Squared error of eight values against codes w dequantized as m * p (MXFP4:
// p = 2^e exactly) or fl32(fl32(m * p) * ts) (NVFP4: p = the E4M3 value),
// accumulated onto acc.  No contraction: y - y^ is rounded before the fma.
template <int FMT>
__device__ __forceinline__ float sse8(const float* v, uint32_t w, float p, float ts, float acc) {
#pragma clang fp contract(off)
  float m[8];
  decode8(w, m);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xh = FMT == FP4_FMT_MXFP4 ? m[i] * p : (m[i] * p) * ts;
    const float d = v[i] - xh;
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc;
}


__device__ __forceinline__ u32x4 mx_enc32(const float* v, uint32_t code) {
  const float sc = e8m0_as_cvt_scale(code);
  return u32x4{enc8_f32(&v[0], sc), enc8_f32(&v[8], sc), enc8_f32(&v[16], sc), enc8_f32(&v[24], sc)};
}

__device__ __forceinline__ float mx_sse32(const float* v, const u32x4& w, uint32_t code) {
  const float p = e8m0_value(code);
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = sse8<FP4_FMT_MXFP4>(&v[8 * t], w[t], p, 0.0f, acc);
  return acc;
}

// MXFP4 block from 32 fp32 values (rotated in place when RN != 0: a group of
// RN blocks, RN = 1, 2 or 4 for 32-, 64- and 128-point rotations); returns the
// E8M0 code and the four code dwords.  RND: stochastic rounding of the exact
// quotients y * 2^-e, element indices base .. base + 31.
template <int RN, int RULE, int RND>
__device__ __forceinline__ uint32_t mx_block_f32(float* v, u32x4& out, uint32_t kb, uint64_t base,
                                                 const QParams& P) {
  if constexpr (RN != 0) rotate_block<32, RN>(v, kb, P);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2(amax)) = exponent field - 127 for a normal amax; subnormal and
  // zero amax clamp to the smallest scale (code 0).
  const uint32_t code = (uint32_t)max((int)((as_u(amax) >> 23) & 0xFFu) - 2, 0);
  if constexpr (RND != 0) {
    const float inv = e8m0_value(254u - code);  // 2^-(code - 127)
    uint32_t w[32];
    sr_words<32>(base, P, w);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= inv;
    out = u32x4{enc8_sr(&v[0], &w[0]), enc8_sr(&v[8], &w[8]), enc8_sr(&v[16], &w[16]),
                enc8_sr(&v[24], &w[24])};
    return code;
  }
  out = mx_enc32(v, code);
  if constexpr (RULE == FP4_SCALE_MSE) {
    if (code < 254u) {
      const u32x4 o1 = mx_enc32(v, code + 1u);
      if (mx_sse32(v, o1, code + 1u) < mx_sse32(v, out, code)) {
        out = o1;
        return code + 1u;
      }
    }
  }
  return code;
}

// MXFP4 block straight from 16 bf16 pairs: |x| orders like its 15 low bits.
__device__ __forceinline__ uint32_t mx_block_bf16(const uint32_t* w, u32x4& out) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  const uint32_t amax_bits = (uint32_t)max(m[0], m[1]);
  const uint32_t code = (uint32_t)max((int)((amax_bits >> 7) & 0xFFu) - 2, 0);
  const float sc = e8m0_as_cvt_scale(code);
  // each call encodes 8 elements (4 input dwords) into one output dword
  out[0] = enc8_bf16(&w[0], sc);
  out[1] = enc8_bf16(&w[4], sc);
  out[2] = enc8_bf16(&w[8], sc);
  out[3] = enc8_bf16(&w[12], sc);
  return code;
}

// MXINT4 block from 32 fp32 values (rotated in place when ROT): the MXFP4
// E8M0 code, elements round(y / 2^e) clipped to +-7 ("Bridging the Gap ...",
// MXINT4).  y * 2^-e is the correctly rounded quotient (a power-of-two factor).
template <int RN>
__device__ __forceinline__ uint32_t mxint_block_f32(float* v, u32x4& out, uint32_t kb,
                                                    const QParams& P) {
  if constexpr (RN != 0) rotate_block<32, RN>(v, kb, P);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t code = (uint32_t)max((int)((as_u(amax) >> 23) & 0xFFu) - 2, 0);
  const float inv = e8m0_value(254u - code);  // 2^-(code - 127)
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= inv;
  out = u32x4{int4_pack8(&v[0]), int4_pack8(&v[8]), int4_pack8(&v[16]), int4_pack8(&v[24])};
  return code;
}

// Tensor-scale constants of one NVFP4 launch.
struct NvTs {
  float ts, inv_ts;
  bool live, small;
};

__device__ __forceinline__ NvTs make_ts(float ts) {
  NvTs t;
  t.ts = ts;
  t.live = ts > 0.0f;
  t.small = ts < 0x1p-100f;
  t.inv_ts = t.live ? 1.0f / ts : 0.0f;
  return t;
}

// NVFP4 block scale from the block's amax: returns the E4M3 code and sets s
// to the decoded scale e4m3 * ts (0 when the tensor scale or the block is 0).
// E4M3 code of t = fl32(h / ts) (h = fl32(amax / 6), or amax / 4 for the
// alternative of Four Over Six).
__device__ __forceinline__ uint32_t nv_code_of(float h, const NvTs& T) {
  const float t = (T.small || h < 0x1p-100f) ? h / T.ts : div_rn(h, T.ts, T.inv_ts);
  return e4m3_rne_sat(t);
}

__device__ __forceinline__ uint32_t nv_scale(float amax, const NvTs& T, float& s) {
  uint32_t code = 0;
  s = 0.0f;
  if (T.live) {
    const float inv6 = 0x1.555556p-3f;  // fl32(1/6)
    const float h = (amax < 0x1p-100f) ? amax / 6.0f : div_rn(amax, 6.0f, inv6);
    code = nv_code_of(h, T);
    s = e4m3_value(code) * T.ts;
  }
  return code;
}

// Eight values of an NVFP4 block -> one dword of codes, q = fl32(v / s)
// rounded to E2M1 (v is overwritten).  For normal scales the quotients are
// formed negated and the eight sign bits flipped afterwards.
// nv_enc8_rs: the normal-scale case (s >= 2^-100) with rs = fl32(1 / s) given.
__device__ __forceinline__ uint32_t nv_enc8_rs(float* v, float s, float rs) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = neg_div_rn(v[i], s, rs);
  return enc8_f32(v, 1.0f) ^ 0x88888888u;  // scale operand 2^0: the quotient is exact
}

__device__ __forceinline__ uint32_t nv_enc8(float* v, float s) {
  if (s == 0.0f) return 0u;
  if (s >= 0x1p-100f) return nv_enc8_rs(v, s, 1.0f / s);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] / s;
  return enc8_f32(v, 1.0f);
}

// NVFP4 block from 16 fp32 values (rotated in place when ROT).
// With ROT the 1/sqrt(16) = 1/4 of the rotation is folded into the divisor
// when the tensor scale is at least 2^-100: every block scale is then at
// least 2^-109, a butterfly sum S that can round to a non-zero code has
// |S| > s, so y = S/4 is a normal float (exact), fl32(S / (4 s)) equals
// fl32(y / s), and max|y| = max|S| / 4 (rounding is monotone).  Smaller
// tensor scales take the division by 4 first, as the definition orders it.
// Codes of 16 values at scale s (v is kept).
__device__ __forceinline__ u32x2 nv_enc16(const float* v, float s) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = v[i];
  return u32x2{nv_enc8(&t[0], s), nv_enc8(&t[8], s)};
}

__device__ __forceinline__ float nv_sse16(const float* v, const u32x2& w, uint32_t code, float ts) {
  const float p = e4m3_value(code);
  return sse8<FP4_FMT_NVFP4>(&v[8], w[1], p, ts, sse8<FP4_FMT_NVFP4>(&v[0], w[0], p, ts, 0.0f));
}

// NVFP4 block under a searching rule (values already rotated and normalised):
// the absmax code c0, then the rule's candidates in order.
template <int RULE>
__device__ __forceinline__ uint32_t nv_block_search(const float* v, float amax, const NvTs& T,
                                                    u32x2& out) {
  float s;
  uint32_t best = nv_scale(amax, T, s);
  out = nv_enc16(v, s);
  if (!T.live) return best;
  float best_e = nv_sse16(v, out, best, T.ts);
  const int c0 = (int)best;
  constexpr int NC = RULE == FP4_SCALE_MSE ? 8 : 1;
  constexpr int kWindow[8] = {1, -1, 2, -2, 3, 4, 5, 6};
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    int c;
    if constexpr (RULE == FP4_SCALE_MSE) c = c0 + kWindow[k];
    else c = (int)nv_code_of(amax * 0.25f, T);  // maximum onto 4
    if (c < 0 || c > 0x7E) continue;
    const u32x2 o = nv_enc16(v, e4m3_value((uint32_t)c) * T.ts);
    const float e = nv_sse16(v, o, (uint32_t)c, T.ts);
    if (e < best_e) {
      best_e = e;
      best = (uint32_t)c;
      out = o;
    }
  }
  return best;
}

// Absmax block scale and nearest rounding of 16 values (rotated already) with
// block maximum amax; the divisor is 4 s when fold (the rotation's 1/4 moved
// into it).
// The common case of nv_scale with no branches: when the block maximum, the
// quotients and the E4M3 block scale are normal and the divisor d (4 s when
// fold) is at least 2^-100, nv_scale and nv_enc8 reduce to these steps (same
// operations, same results).  Returns whether the case applies.
// nv_code_fast: the E4M3 code of that case, with h = fl32(amax / 6) and
// t = min(fl32(h / ts), 448) (a meaningless code when t < 2^-6).
__device__ __forceinline__ uint32_t nv_code_fast(float amax, const NvTs& T, float& h, float& t) {
  h = div_rn(amax, 6.0f, 0x1.555556p-3f);
  t = fminf(div_rn(h, T.ts, T.inv_ts), 448.0f);
  uint32_t u = as_u(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);
}

__device__ __forceinline__ bool nv_scale_fast(float amax, bool fold, const NvTs& T, uint32_t& code,
                                              float& d) {
  float h, t;
  code = nv_code_fast(amax, T, h, t);
  const float s = as_f((((code >> 3) + 120u) << 23) | ((code & 7u) << 20)) * T.ts;
  d = fold ? 4.0f * s : s;
  return T.live && !T.small && amax >= 0x1p-100f && h >= 0x1p-100f && t >= 0x1p-6f &&
         d >= 0x1p-100f;
}

__device__ __forceinline__ uint32_t nv_encode_amax(float* v, float amax, bool fold, const NvTs& T,
                                                   u32x2& out) {
  // branch-free when every lane of the wave takes the common case, with one
  // reciprocal per block
  uint32_t fcode;
  float fd;
  const bool fast = nv_scale_fast(amax, fold, T, fcode, fd);
  if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
    const float rd = 1.0f / fd;
    out[0] = nv_enc8_rs(&v[0], fd, rd);
    out[1] = nv_enc8_rs(&v[8], fd, rd);
    return fcode;
  }
  float s;
  const uint32_t code = nv_scale(amax, T, s);
  const float d = fold ? 4.0f * s : s;
  out[0] = nv_enc8(&v[0], d);
  out[1] = nv_enc8(&v[8], d);
  return code;
}

template <int ROT, int RULE, int RND>
__device__ __forceinline__ uint32_t nv_block(float* v, const NvTs& T, u32x2& out, uint32_t kb,
                                             uint64_t base, const QParams& P) {
  if constexpr (RULE != FP4_SCALE_ABSMAX) {
    if constexpr (ROT != 0) rotate_block<16, 1>(v, kb, P);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    return nv_block_search<RULE>(v, amax, T, out);
  }
  const bool fold = ROT && !T.small;
  if constexpr (ROT != 0) {
    if (P.any_sign) apply_signs<16>(v, P.signs[0]);
    fwht<16>(v);
    if (T.small) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] *= 0.25f;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (fold) amax *= 0.25f;
  if constexpr (RND == 0) return nv_encode_amax(v, amax, fold, T, out);
  // stochastic rounding of the exact quotients fl32(y / s)
  float s;
  const uint32_t code = nv_scale(amax, T, s);
  const float d = fold ? 4.0f * s : s;
  if (d == 0.0f) {
    out = u32x2{0u, 0u};
    return code;
  }
  if (d >= 0x1p-100f) {
    const float rd = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = div_rn(v[i], d, rd);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] / d;
  }
  uint32_t w[16];
  sr_words<16>(base, P, w);
  out = u32x2{enc8_sr(&v[0], &w[0]), enc8_sr(&v[8], &w[8])};
  return code;
}

// NVINT4 block from 16 fp32 values (rotated in place when ROT): E4M3 code of
// (amax / 7) / ts, elements round(fl32(y / s)) clipped to +-7.
template <int ROT>
__device__ __forceinline__ uint32_t nvint_block(float* v, const NvTs& T, u32x2& out, uint32_t kb,
                                                const QParams& P) {
  if constexpr (ROT != 0) rotate_block<16, 1>(v, kb, P);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t code = 0;
  float s = 0.0f;
  if (T.live) {
    code = nv_code_of(amax / 7.0f, T);
    s = e4m3_value(code) * T.ts;
  }
  if (s == 0.0f) {
    out = u32x2{0u, 0u};
    return code;
  }
  if (s >= 0x1p-100f) {
    const float rs = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = div_rn(v[i], s, rs);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] / s;
  }
  out = u32x2{int4_pack8(&v[0]), int4_pack8(&v[8])};
  return code;
}

// Unpack a block held as raw 16-byte chunks into fp32.
template <int XDT, int G>
__device__ __forceinline__ void unpack(const u32x4* c, float* v) {
  if constexpr (XDT == FP4_DT_BF16) {
#pragma unroll
    for (int i = 0; i < G / 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_lo(c[i][j]);
        v[8 * i + 2 * j + 1] = bf16_hi(c[i][j]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < G / 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = as_f(c[i][j]);
  }
}

// NVFP4 absmax / nearest blocks whose values were prepared ahead (bf16
// unpacked; with ROT signed and put through the butterflies but not yet
// divided by 4) with their maximum am, for the single-pass kernel, which
// prepares them before the exchange.  nv_prep_block prepares one block;
// nv_encode_prepped encodes one as nv_block would; nv_encode_tiles_tab
// encodes N blocks (one per tile of the wave) in one branch-free sequence when
// every block of the wave takes nv_scale_fast's common case, and returns
// false (wave-uniform, nothing done) otherwise.  (The two-pass kernel keeps
// its per-tile path: holding the fp32 blocks of both of its tiles halves its
// occupancy, measured 0.4-0.7 us slower per 4096 x 4096 launch.)
template <int ROT>
__device__ __forceinline__ void nv_prep_block(const u32x4* c, float* v, float& am, const QParams& P) {
  unpack<FP4_DT_BF16, 16>(c, v);
  if constexpr (ROT != 0) {
    if (P.any_sign) apply_signs<16>(v, P.signs[0]);
    fwht<16>(v);
  }
  am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
}

template <int ROT>
__device__ __forceinline__ uint32_t nv_encode_prepped(float* v, float am, const NvTs& T, u32x2& out) {
  if (ROT != 0 && T.small) {  // nv_block divides by 4 first here
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] *= 0.25f;
      a = fmaxf(a, fabsf(v[i]));
    }
    return nv_encode_amax(v, a, false, T, out);
  }
  return nv_encode_amax(v, ROT != 0 ? am * 0.25f : am, ROT != 0, T, out);
}

// Divisor table of one launch for nv_encode_tiles_tab: entry c holds
// d = e4m3(c) * ts (times 4 with ROT, the fold) and fl32(1 / d), the values
// nv_scale_fast and nv_encode_amax derive per block.
template <int ROT>
__device__ __forceinline__ void nv_divisor_entry(uint32_t c, float ts, float (&tab)[128][2]) {
  const float s = e4m3_value(c) * ts;
  const float d = ROT != 0 ? 4.0f * s : s;
  tab[c][0] = d;
  tab[c][1] = 1.0f / d;
}

// The common case for N blocks with the block divisors and their reciprocals
// looked up in the launch's divisor table: the values nv_scale_fast and
// nv_encode_amax would compute per block.
template <int ROT, int N>
__device__ __forceinline__ bool nv_encode_tiles_tab(float (&v)[N][16], const float (&am)[N],
                                                    const NvTs& T, const float (&tab)[128][2],
                                                    uint32_t (&code)[N], u32x2 (&out)[N]) {
  float d[N], rd[N];
  bool fast = T.live && !T.small;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const float a = ROT != 0 ? am[u] * 0.25f : am[u];
    float h, t;
    code[u] = nv_code_fast(a, T, h, t);
    const uint32_t c = min(code[u], 127u);
    d[u] = tab[c][0];
    rd[u] = tab[c][1];
    fast &= a >= 0x1p-100f && h >= 0x1p-100f && t >= 0x1p-6f && d[u] >= 0x1p-100f;
  }
  if (__builtin_amdgcn_ballot_w64(!fast) != 0) return false;
#pragma unroll
  for (int u = 0; u < N; ++u)
    out[u] = u32x2{nv_enc8_rs(&v[u][0], d[u], rd[u]), nv_enc8_rs(&v[u][8], d[u], rd[u])};
  return true;
}

__device__ __forceinline__ void store_mx_scale(uint8_t* __restrict__ scales, int64_t r, int64_t kb,
                                               int64_t nb, int64_t kchunks, int gemm_layout,
                                               uint32_t code) {
  const int64_t off = gemm_layout ? mx_gemm_scale_offset(r, kb, kchunks) : r * nb + kb;
  scales[off] = (uint8_t)code;
}

// Quantize the block held in chunks c: codes in out (four dwords for MXFP4,
// the first two for NVFP4), scale code returned.
// Block kb of row r (element index r * cols + kb * G, for stochastic rounding).
template <int FMT, int XDT, int ROT, int RULE, int RND>
__device__ __forceinline__ uint32_t compute_block(const u32x4* c, const NvTs& T, u32x4& out,
                                                  uint32_t r, uint32_t kb, const QParams& P) {
  constexpr int G = fmt_block(FMT);
  const uint64_t base = (uint64_t)r * (uint64_t)P.cols + (uint64_t)kb * G;
  if constexpr (FMT == FP4_FMT_MXINT4) {
    float v[32];
    unpack<XDT, 32>(c, v);
    return mxint_block_f32<ROT>(v, out, kb, P);
  } else if constexpr (FMT == FP4_FMT_NVINT4) {
    float v[16];
    unpack<XDT, 16>(c, v);
    u32x2 o;
    const uint32_t code = nvint_block<ROT>(v, T, o, kb, P);
    out = u32x4{o[0], o[1], 0u, 0u};
    return code;
  } else if constexpr (FMT == FP4_FMT_MXFP4) {
    if constexpr (XDT == FP4_DT_BF16 && !ROT && RULE == FP4_SCALE_ABSMAX && RND == 0) {
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * i + j] = c[i][j];
      return mx_block_bf16(w, out);
    } else {
      float v[32];
      unpack<XDT, 32>(c, v);
      return mx_block_f32<ROT, RULE, RND>(v, out, kb, base, P);
    }
  } else {
    float v[16];
    unpack<XDT, 16>(c, v);
    u32x2 o;
    const uint32_t code = nv_block<ROT, RULE, RND>(v, T, o, kb, base, P);
    out = u32x4{o[0], o[1], 0u, 0u};
    return code;
  }
}

// Store the codes and scale of block (r, kb).
template <int FMT>
__device__ __forceinline__ void store_block(const u32x4& out, uint32_t code, int64_t r, int64_t kb,
                                            int64_t nb, uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales, int64_t kchunks,
                                            int gemm_layout, uint32_t tiled) {
  // tiled is uniform: a branch, so the row-major path costs no extra VALU
  if constexpr (fmt_mx(FMT)) {
    if (tiled)
      *reinterpret_cast<u32x4*>(codes + code_offset(r, kb * 16, nb * 16, true)) = out;
    else
      *reinterpret_cast<u32x4*>(codes + r * (nb * 16) + kb * 16) = out;
    store_mx_scale(scales, r, kb, nb, kchunks, gemm_layout, code);
  } else {
    if (tiled)
      *reinterpret_cast<u32x2*>(codes + code_offset(r, kb * 8, nb * 8, true)) = u32x2{out[0], out[1]};
    else
      *reinterpret_cast<u32x2*>(codes + r * (nb * 8) + kb * 8) = u32x2{out[0], out[1]};
    scales[r * nb + kb] = (uint8_t)code;
  }
}

template <int FMT, int XDT, int ROT, int RULE, int RND>
__device__ __forceinline__ void quantize_block(const u32x4* c, const NvTs& T, int64_t r, int64_t kb,
                                               int64_t nb, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales, int64_t kchunks,
                                               int gemm_layout, const QParams& P) {
  u32x4 out;
  const uint32_t code = compute_block<FMT, XDT, ROT, RULE, RND>(c, T, out, (uint32_t)r, (uint32_t)kb, P);
  store_block<FMT>(out, code, r, kb, nb, codes, scales, kchunks, gemm_layout, P.tiled);
}

// Max of a workgroup (all threads must call); valid in every thread.
__device__ __forceinline__ float wg_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kThreads / 64];
  const int wave = (int)wave_index();
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// NVFP4 tensor scale for this launch: either given (*gs), or reduced from the
// amax pass's partial maxima (workgroup 0 then publishes it to *gs).
// The tensor scale maps the tensor maximum onto 448 * qmax: 2688 for the E2M1
// element, 3136 for INT4.
template <int FMT>
__device__ __forceinline__ NvTs nv_launch_ts(float* __restrict__ gs,
                                             const float* __restrict__ partials, int npart) {
  if (npart <= 0) return make_ts(*gs);
  float m = 0.0f;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = fmaxf(m, partials[i]);
  m = wg_max(m);
  const float ts = m / (448.0f * fmt_qmax(FMT));
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs = ts;
  return make_ts(ts);
}

// ----------------------------------------------------------- tiled kernel
// Requires nb % 64 == 0.  Wave w of the grid-stride loop owns row r, blocks
// [64 g, 64 g + 64).
template <int FMT, int XDT, int ROT, int RULE, int RND>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(
    const void* __restrict__ x, int64_t ldx, uint32_t rows, uint32_t nb,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t kchunks, int gemm_layout,
    float* __restrict__ gs, const float* __restrict__ partials, int npart, QParams P) {
  constexpr int G = fmt_block(FMT);
  constexpr int ES = XDT == FP4_DT_BF16 ? 2 : 4;
  constexpr int BB = G * ES;       // bytes per block
  constexpr int CH = BB / 16;      // 16-byte chunks per block
  constexpr int STRIDE = BB + 16;  // padded LDS stride: conflict-free 16-byte reads
  __shared__ __attribute__((aligned(16))) uint8_t lds[kThreads / 64][64 * STRIDE];

  NvTs T{};
  if constexpr (!fmt_mx(FMT)) T = nv_launch_ts<FMT>(gs, partials, npart);

  const int lane = threadIdx.x & 63, wave = (int)wave_index();
  const uint32_t groups = nb / 64;
  const uint32_t tiles = rows * groups;
  uint8_t* l = lds[wave];
  for (uint32_t base = blockIdx.x * (kThreads / 64); base < tiles; base += gridDim.x * (kThreads / 64)) {
    const uint32_t tile = base + wave;
    const bool active = tile < tiles;
    const uint32_t r = active ? tile / groups : 0;
    const uint32_t g = active ? tile - r * groups : 0;
    if (active) {
      const uint8_t* src = static_cast<const uint8_t*>(x) + ((int64_t)r * ldx + (int64_t)g * 64 * G) * ES;
      u32x4 t[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) t[j] = *reinterpret_cast<const u32x4*>(src + (j * 64 + lane) * 16);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = j * 64 + lane;
        *reinterpret_cast<u32x4*>(l + (c / CH) * STRIDE + (c % CH) * 16) = t[j];
      }
    }
    __syncthreads();
    if (active) {
      u32x4 c[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) c[k] = *reinterpret_cast<const u32x4*>(l + lane * STRIDE + k * 16);
      quantize_block<FMT, XDT, ROT, RULE, RND>(c, T, r, (int64_t)g * 64 + lane, nb, codes, scales,
                                               kchunks, gemm_layout, P);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- bf16 tile kernels
// bf16 input, any shape (cols a multiple of the block size, rows 16-byte
// aligned).  Every quantization block is computed by one lane, in registers;
// the input arrives with fully coalesced 16-byte non-temporal loads and is
// transposed through a padded per-wave LDS buffer (stride block + 16 bytes, so
// both the scattered writes and the per-lane block reads are conflict-free).
// Only the wave itself touches its LDS buffer: a wave-scope fence and wave
// barrier order the writes before the reads, with no workgroup barrier.
// Lanes past the edge of the tensor load an in-bounds chunk again and store
// nothing.
__device__ __forceinline__ u32x4 load_nt16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void unpack8_bf16(const u32x4& w, float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(w[j]);
    v[2 * j + 1] = bf16_hi(w[j]);
  }
}

// NVFP4 tensor scale for one wave, in two steps so that the loads of the
// partial maxima (or of the given scale) are issued before the tile loads and
// waiting for them never waits for the tile: nv_ts_issue loads the given
// *gs, or the amax pass's partials (npart <= kAmaxGrid = 8 x 64: eight loads
// per lane; indices past the end re-read the last partial, which leaves the
// maximum unchanged); nv_ts_finish reduces them (wave 0 of workgroup 0
// publishes the computed scale to *gs).
struct NvTsLoads {
  float p[kAmaxGrid / 64];
};

__device__ __forceinline__ NvTsLoads nv_ts_issue(const float* __restrict__ gs,
                                                 const float* __restrict__ partials, int npart) {
  NvTsLoads L;
  if (npart <= 0) {
    L.p[0] = *gs;
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kAmaxGrid / 64; ++k) L.p[k] = partials[min(lane + 64 * k, npart - 1)];
  }
  return L;
}

template <int FMT>
__device__ __forceinline__ NvTs nv_ts_finish(const NvTsLoads& L, float* __restrict__ gs, int npart,
                                             bool publish) {
  if (npart <= 0) return make_ts(L.p[0]);
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kAmaxGrid / 64; ++k) m = fmaxf(m, L.p[k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float ts = m / (448.0f * fmt_qmax(FMT));
  if (publish && (threadIdx.x & 63) == 0) *gs = ts;
  return make_ts(ts);
}

// Row tiles (row-major scales: NVFP4, and MXFP4 when asked for row-major
// scales).  Wave tile (r, w) = blocks [64 w, 64 w + 64) of row r; each wave
// issues the loads of TPW tiles before any arithmetic, then runs them one by
// one through its LDS buffer.  The scale bytes of a wave tile are 64
// consecutive bytes of its row.
// LDS bytes of a quant_rows workgroup.
template <int FMT>
constexpr int rows_lds_bytes() {
  return (kThreads / 64) * 64 * (fmt_block(FMT) * 2 + 16);
}

// Body of the row-tile kernel for workgroup bid of nbid, LDS at lds.
template <int FMT, int ROT, int TPW, int RULE, int RND>
__device__ __forceinline__ void quant_rows_body(
    uint8_t* lds, uint32_t bid, uint32_t nbid, const uint8_t* __restrict__ x, int64_t ldx_bytes,
    uint32_t rows, uint32_t nb, uint32_t wpr, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t kchunks, int gemm_layout, float* __restrict__ gs,
    const float* __restrict__ partials, int npart, const QParams& P) {
  constexpr int G = fmt_block(FMT);
  constexpr int BB = G * 2;        // bytes per block
  constexpr int CH = BB / 16;      // 16-byte chunks per block
  constexpr int STRIDE = BB + 16;  // padded LDS stride
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_index();
  const uint32_t tiles = rows * wpr;
  const uint32_t step = nbid * (kThreads / 64) * TPW;
  uint32_t t0 = (bid * (kThreads / 64) + wave) * TPW;
  if (t0 >= tiles) return;
  const uint32_t last_chunk = nb * CH - 1;
  uint8_t* l = lds + wave * (64 * STRIDE);
  u32x4 t[TPW][CH];
  auto load = [&](uint32_t first) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const uint32_t tile = min(first + u, tiles - 1);
      const uint32_t r = tile / wpr, w = tile - r * wpr;
      const uint8_t* row = x + (int64_t)r * ldx_bytes;
#pragma unroll
      for (int j = 0; j < CH; ++j)
        t[u][j] = load_nt16(row + (int64_t)min(w * 64 * CH + j * 64 + lane, last_chunk) * 16);
    }
  };
  NvTsLoads tsl{};
  if constexpr (!fmt_mx(FMT)) tsl = nv_ts_issue(gs, partials, npart);
  load(t0);
  NvTs T{};
  if constexpr (!fmt_mx(FMT)) T = nv_ts_finish<FMT>(tsl, gs, npart, bid == 0 && wave == 0);
  for (;;) {
    // all tiles computed before any store, so no store sits between a tile
    // load and the wait for it
    u32x4 out[TPW];
    uint32_t code[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = j * 64 + lane;
        *reinterpret_cast<u32x4*>(l + (c / CH) * STRIDE + (c % CH) * 16) = t[u][j];
      }
      wave_lds_sync();
      u32x4 c[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) c[k] = *reinterpret_cast<const u32x4*>(l + lane * STRIDE + k * 16);
      wave_lds_sync();
      const uint32_t tile_u = min(t0 + u, tiles - 1);
      const uint32_t r_u = tile_u / wpr;
      code[u] = compute_block<FMT, FP4_DT_BF16, ROT, RULE, RND>(c, T, out[u], r_u,
                                                                (tile_u - r_u * wpr) * 64 + lane, P);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const uint32_t tile = t0 + u;
      const uint32_t r = tile / wpr, w = tile - r * wpr;
      const uint32_t kb = w * 64 + lane;
      if (tile < tiles && kb < nb)
        store_block<FMT>(out[u], code[u], r, kb, nb, codes, scales, kchunks, gemm_layout, P.tiled);
    }
    t0 += step;
    if (t0 >= tiles) break;
    load(t0);
  }
}

template <int FMT, int ROT, int TPW, int RULE, int RND>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t rows, uint32_t nb, uint32_t wpr,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t kchunks, int gemm_layout,
    float* __restrict__ gs, const float* __restrict__ partials, int npart, QParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[rows_lds_bytes<FMT>()];
  quant_rows_body<FMT, ROT, TPW, RULE, RND>(lds, blockIdx.x, gridDim.x, x, ldx_bytes, rows, nb, wpr,
                                            codes, scales, kchunks, gemm_layout, gs, partials,
                                            npart, P);
}

// NVFP4 / NVINT4 with the tensor scale computed in the same launch, for a
// tensor small enough to sit in the registers of one co-resident grid.  Each
// wave loads all of its wave tiles (tile gw + u * waves for u < TPW), moves
// them into per-lane blocks through its LDS buffer and takes the maximum of
// the block values (rotated with ROT, as the encoder rotates them); the
// workgroups exchange their maxima; then every workgroup encodes its tiles
// from registers.  The input crosses HBM once instead of twice (maximum
// pass, then encode pass).
//
// Exchange: xchg[0] is a call number E - 1, then (from xchg + 16) one 64-bit
// slot per workgroup.  A workgroup reads E at its start, stores (E, its
// maximum) to its slot in one single-copy-atomic 64-bit store, and polls all
// slots until each carries E; the values are then this call's maxima, so no
// other ordering is needed.  Workgroup 0 finally stores E to xchg[0].  The
// region must be zero before its first use (later calls find it as the last
// call left it).  The host caps the grid at one workgroup per CU, so the
// whole grid is resident at once when no other grid-synchronising kernel
// shares the device.  A wait that outlasts its bound (seconds) gives up: that
// workgroup encodes with a NaN tensor scale (all-zero codes), stores NaN
// to *gs and sets xchg[1] (the give-up flag); the region then needs zeroing
// again.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kMaxDevices = 64;
constexpr uint32_t kExchangeSpin = 1u << 22;

template <int FMT, int ROT, int TPW, int RULE, int RND>
__global__ __launch_bounds__(kFusedThreads) void quant_nv_fused_kernel(
    const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t rows, uint32_t nb, uint32_t wpr,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gs,
    uint32_t* __restrict__ xchg, QParams P) {
  constexpr int CH = 2;            // 16-byte chunks of a 16-element bf16 block
  constexpr int STRIDE = 32 + 16;  // padded LDS stride
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFusedWaves][64 * STRIDE];
  __shared__ float red[kFusedWaves];
  __shared__ float ts_shared;
  __shared__ float dtab[128][2];
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_index();
  const uint32_t tiles = rows * wpr;
  const uint32_t waves = gridDim.x * kFusedWaves;
  const uint32_t gw = blockIdx.x * kFusedWaves + wave;
  const uint32_t last_chunk = nb * CH - 1;
  uint64_t* slots = reinterpret_cast<uint64_t*>(xchg + 16);
  uint8_t* l = lds[wave];

  uint32_t E = 0;
  if (wave == 0) E = __hip_atomic_load(&xchg[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  u32x4 c[TPW][CH];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const uint32_t tile = min(gw + u * waves, tiles - 1);
    const uint32_t r = tile / wpr, w = tile - r * wpr;
    const uint8_t* row = x + (int64_t)r * ldx_bytes;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      c[u][j] = load_nt16(row + (int64_t)min(w * 64 * CH + j * 64 + lane, last_chunk) * 16);
  }
  // Maximum over the wave's blocks.  Tiles past the end re-read the last
  // tile, which leaves the maximum unchanged; lanes past the row end hold
  // re-read chunks, not blocks of the tensor, and are left out.  Plain: the
  // largest magnitude's bf16 bits, as the separate maximum pass takes it.
  // PREP (NVFP4, absmax, nearest, 4 tiles per wave): phase 1 also keeps each
  // block's fp32 values (rotated, not yet divided by 4) and their maximum, so
  // the encoding after the exchange starts from them.
  constexpr bool PREP = FMT == FP4_FMT_NVFP4 && RULE == FP4_SCALE_ABSMAX && RND == 0 && TPW == 4;
  float vv[PREP ? TPW : 1][16];
  float am[PREP ? TPW : 1];
  uint32_t mb = 0;
  float mf = 0.0f;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int q = j * 64 + lane;
      *reinterpret_cast<u32x4*>(l + (q / CH) * STRIDE + (q % CH) * 16) = c[u][j];
    }
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < CH; ++k) c[u][k] = *reinterpret_cast<const u32x4*>(l + lane * STRIDE + k * 16);
    wave_lds_sync();
    uint32_t bm = 0;  // plain: the block's largest magnitude as bf16 bits
    if constexpr (ROT == 0) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        u16x2 m = __builtin_bit_cast(u16x2, c[u][k][0] & 0x7FFF7FFFu);
#pragma unroll
        for (int e = 1; e < 4; ++e)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, c[u][k][e] & 0x7FFF7FFFu));
        bm = max(bm, (uint32_t)max(m[0], m[1]));
      }
      if constexpr (PREP) {
        // the block maximum from the same bits, computed here so that the
        // encoding after the exchange starts from it (it differs from a
        // float maximum only for NaN inputs, which the contract excludes)
        unpack<FP4_DT_BF16, 16>(c[u], vv[u]);
        am[u] = as_f(bm << 16);
      }
    } else if constexpr (PREP) {
      nv_prep_block<ROT>(c[u], vv[u], am[u], P);
    }
    const uint32_t tile = min(gw + u * waves, tiles - 1);
    if ((tile - (tile / wpr) * wpr) * 64 + lane >= nb) continue;
    if constexpr (PREP && ROT != 0) {
      mf = fmaxf(mf, am[u]);
    } else if constexpr (ROT == 0) {
      mb = max(mb, bm);
    } else {
      float v[16];
      unpack<FP4_DT_BF16, 16>(c[u], v);
      if (P.any_sign) apply_signs<16>(v, P.signs[0]);
      fwht<16>(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) mf = fmaxf(mf, fabsf(v[i]));
    }
  }
  float m = ROT ? mf : as_f(mb << 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();

  if (wave == 0) {
    float wm = red[0];
#pragma unroll
    for (int i = 1; i < kFusedWaves; ++i) wm = fmaxf(wm, red[i]);
    if (ROT) wm *= 0.25f;  // 1/sqrt(16), exact
    if (lane == 0)
      __hip_atomic_store(&slots[blockIdx.x], ((uint64_t)E << 32) | __builtin_bit_cast(uint32_t, wm),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
    float t = 0.0f;
    for (uint32_t n = 0;; ++n) {
      bool mine = true;
      t = 0.0f;
      for (uint32_t i = lane; i < gridDim.x; i += 64) {
        const uint64_t v = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine &= (uint32_t)(v >> 32) == E;
        t = fmaxf(t, __builtin_bit_cast(float, (uint32_t)v));
      }
      if (__builtin_amdgcn_ballot_w64(!mine) == 0) break;
      if (n == kExchangeSpin) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t = fmaxf(t, __shfl_xor(t, off, 64));
    const float ts = ok ? t / (448.0f * fmt_qmax(FMT)) : __builtin_nanf("");
    if constexpr (PREP) {
      nv_divisor_entry<ROT>(lane, ts, dtab);
      nv_divisor_entry<ROT>(lane + 64, ts, dtab);
    }
    if (lane == 0) {
      ts_shared = ts;
      if (blockIdx.x == 0 || !ok) *gs = ts;
      // the give-up flag (word 1 of the region): NaN in *gs alone could be
      // overwritten by workgroup 0's finite scale
      if (!ok) __hip_atomic_store(&xchg[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (blockIdx.x == 0) __hip_atomic_store(&xchg[0], E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const NvTs T = make_ts(ts_shared);

  if constexpr (PREP) {
    // Common case for all tiles at once, straight-line so that the tiles'
    // steps interleave: every block of every tile of the wave normal (tiles
    // past the end and lanes past a row's end hold re-read tensor values,
    // computed and not stored).
    uint32_t fc[TPW];
    u32x2 fo[TPW];
    if (nv_encode_tiles_tab<ROT, TPW>(vv, am, T, dtab, fc, fo)) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const uint32_t tile = gw + u * waves;
        const uint32_t r = tile / wpr, w = tile - r * wpr;
        const uint32_t kb = w * 64 + lane;
        if (tile < tiles && kb < nb)
          store_block<FMT>(u32x4{fo[u][0], fo[u][1], 0u, 0u}, fc[u], r, kb, nb, codes, scales, 0, 0, P.tiled);
      }
      return;
    }
  }

#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const uint32_t tile = gw + u * waves;
    if (tile >= tiles) break;
    const uint32_t r = tile / wpr, w = tile - r * wpr;
    const uint32_t kb = w * 64 + lane;
    u32x4 out;
    uint32_t code;
    if constexpr (PREP) {
      // the steps of nv_block after its rotation and maximum (the uncommon
      // cases; the common one ran above for all tiles at once)
      u32x2 o;
      code = nv_encode_prepped<ROT>(vv[u], am[u], T, o);
      out = u32x4{o[0], o[1], 0u, 0u};
    } else {
      code = compute_block<FMT, FP4_DT_BF16, ROT, RULE, RND>(c[u], T, out, r, kb, P);
    }
    if (kb < nb) store_block<FMT>(out, code, r, kb, nb, codes, scales, 0, 0, P.tiled);
  }
}

// MXFP4 with GEMM-layout scales.  A workgroup tile is 32 rows x 256 columns,
// exactly the rows and K range of one 256-byte scale tile, so the workgroup
// writes whole scale tiles (from one CU, merged in one L2) instead of
// scattering bytes over tiles that other workgroups share.  Wave w takes rows
// 8w .. 8w + 7 of the tile; load j brings rows 2j, 2j + 1 (512 bytes each);
// after the LDS transpose lane l holds block l % 8 of row l / 8, and the
// codes of each row (8 blocks) are 128 contiguous bytes.
constexpr int kMxGemmLds = (kThreads / 64) * 64 * (64 + 16);

template <int FMT, int ROT, int RULE, int RND>
__device__ __forceinline__ void quant_mx_gemm_body(
    uint8_t* lds, uint32_t bid, uint32_t nbid, const uint8_t* __restrict__ x, int64_t ldx_bytes,
    uint32_t rows, uint32_t nb, uint32_t kcs, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t kchunks, const QParams& P) {
  constexpr int STRIDE = 64 + 16;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_index();
  const uint32_t tiles = ((rows + 31) / 32) * kcs;
  const uint32_t cpr = nb * 4;  // 16-byte chunks per row
  uint8_t* l = lds + wave * (64 * STRIDE);
  for (uint32_t tile = bid; tile < tiles; tile += nbid) {
    const uint32_t rt = tile / kcs, kc = tile - rt * kcs;
    const uint32_t r0 = rt * 32 + wave * 8;
    u32x4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t r = min(r0 + 2 * j + (lane >> 5), rows - 1);
      const uint32_t q = min(kc * 32 + (lane & 31), cpr - 1);
      t[j] = load_nt16(x + (int64_t)r * ldx_bytes + (int64_t)q * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = j * 64 + lane;  // row c / 32 of the wave, chunk c % 32
      const int blk = (c >> 5) * 8 + ((c & 31) >> 2);
      *reinterpret_cast<u32x4*>(l + blk * STRIDE + (c & 3) * 16) = t[j];
    }
    wave_lds_sync();
    u32x4 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = *reinterpret_cast<const u32x4*>(l + lane * STRIDE + k * 16);
    wave_lds_sync();
    const uint32_t r = r0 + (lane >> 3), kb = kc * 8 + (lane & 7);
    if (r < rows && kb < nb)
      quantize_block<FMT, FP4_DT_BF16, ROT, RULE, RND>(c, NvTs{}, r, kb, nb, codes, scales, kchunks, 1, P);
  }
}

template <int FMT, int ROT, int RULE, int RND>
__global__ __launch_bounds__(kThreads) void quant_mx_gemm_kernel(
    const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t rows, uint32_t nb, uint32_t kcs,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t kchunks, QParams P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMxGemmLds];
  quant_mx_gemm_body<FMT, ROT, RULE, RND>(lds, blockIdx.x, gridDim.x, x, ldx_bytes, rows, nb, kcs,
                                          codes, scales, kchunks, P);
}

// NVFP4 tensor amax over bf16 input in the same wave tiles, 16 waves per
// workgroup, one partial maximum per workgroup.  Rotated: the maximum of the
// block-Hadamard outputs (8-point transform in registers, then the cross-lane
// stage; the exact 1/4 is applied to the final maximum).
constexpr int kAmaxThreads = 1024;

// Body for workgroup bid of nbid with NW waves; red: NW floats of LDS.
template <bool ROT, int NW>
__device__ __forceinline__ void amax_chunk_body(float* red, uint32_t bid, uint32_t nbid,
                                                const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                uint32_t rows, uint32_t cpr, uint32_t wpr,
                                                float* __restrict__ partials, uint32_t sign_mask) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_index();
  const uint32_t tiles = rows * wpr;
  const uint32_t step = nbid * NW;
  uint32_t mb = 0;   // plain: max of |x| bf16 bits
  float mf = 0.0f;   // rotated: max of |H x| before the 1/4
  for (uint32_t tile = bid * NW + wave; tile < tiles; tile += step) {
    const uint32_t r = tile / wpr;
    const uint32_t q0 = (tile - r * wpr) * 256 + lane;
    const uint8_t* row = x + (int64_t)r * ldx_bytes;
    u32x4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = load_nt16(row + (int64_t)min(q0 + 64 * j, cpr - 1) * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (q0 + 64 * j >= cpr) t[j] = u32x4{0u, 0u, 0u, 0u};  // past the row end
      if constexpr (!ROT) {
        u16x2 m = __builtin_bit_cast(u16x2, t[j][0] & 0x7FFF7FFFu);
#pragma unroll
        for (int k = 1; k < 4; ++k)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, t[j][k] & 0x7FFF7FFFu));
        mb = max(mb, (uint32_t)max(m[0], m[1]));
      } else {
        float v[8];
        unpack8_bf16(t[j], v);
        // the lane's 8 elements are positions 8 (lane & 1) .. + 7 of the 16-group
        if (sign_mask) apply_signs<8>(v, sign_mask >> (8 * (lane & 1)));
        fwht<8>(v);
        fwht_lane_stage<1>(v, lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) mf = fmaxf(mf, fabsf(v[i]));
      }
    }
  }
  float m = ROT ? mf : as_f(mb << 16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = fmaxf(r, red[i]);
    partials[bid] = ROT ? r * 0.25f : r;  // 1/sqrt(16), exact
  }
}

template <bool ROT>
__global__ __launch_bounds__(kAmaxThreads) void amax_chunk_kernel(const uint8_t* __restrict__ x,
                                                                  int64_t ldx_bytes, uint32_t rows,
                                                                  uint32_t cpr, uint32_t wpr,
                                                                  float* __restrict__ partials,
                                                                  uint32_t sign_mask) {
  __shared__ float red[kAmaxThreads / 64];
  amax_chunk_body<ROT, kAmaxThreads / 64>(red, blockIdx.x, gridDim.x, x, ldx_bytes, rows, cpr, wpr,
                                          partials, sign_mask);
}

// ---------------------------------------------------------- grouped launch
// Several quantizations in one launch: segment s owns workgroups
// [first[s], first[s] + nwg) and runs one of the three bodies above (MXFP4 /
// MXINT4 GEMM-layout tiles, row tiles, or the NVFP4 / NVINT4 tensor-maximum
// pass with four waves per workgroup) on its own tensor, with the work split
// of that body's own launch.  One ramp-up and one drain for the whole group
// instead of one per tensor.
constexpr int kSegMxGemm = 0, kSegRows = 1, kSegAmax = 2;
constexpr int kBatchSegs = 16;
constexpr int kBatchLds = kMxGemmLds > rows_lds_bytes<FP4_FMT_MXFP4>()
                              ? kMxGemmLds
                              : rows_lds_bytes<FP4_FMT_MXFP4>();
static_assert(kBatchLds >= rows_lds_bytes<FP4_FMT_NVFP4>(), "LDS of the grouped kernel");

constexpr uint32_t seg_sel(int kind, int fmt, int rot) {
  return (uint32_t)kind | ((uint32_t)fmt << 4) | ((uint32_t)rot << 8);
}

struct BatchSeg {
  const uint8_t* x;
  uint8_t* codes;
  uint8_t* scales;
  float* gs;
  float* partials;  // amax: written; rows (NVFP4 / NVINT4): read when npart > 0
  int64_t ldx_bytes;
  int64_t kchunks;
  uint32_t nwg;
  uint32_t rows, nb;
  uint32_t aux;     // kcs (GEMM-layout tiles), wpr (row tiles), cpr (amax)
  uint32_t aux2;    // wpr (amax)
  int32_t npart;
  uint32_t sel;
  QParams P;
};

struct BatchArgs {
  uint32_t nseg;
  // first workgroup of each segment, contiguous so that a workgroup finds its
  // segment in one or two scalar cache lines instead of one line per segment
  // (2.2 us less per call of eight 4096 x 4096 jobs)
  uint32_t first[kBatchSegs];
  uint32_t pad[3];
  BatchSeg seg[kBatchSegs];
};

// NV_ROWS: only NVFP4 / NVINT4 row-tile segments (the second launch), so the
// kernel needs that body's registers and LDS alone.
template <bool NV_ROWS>
__global__ __launch_bounds__(kThreads) void quant_batch_kernel(BatchArgs A) {
  __shared__ __attribute__((aligned(16)))
  uint8_t lds[NV_ROWS ? rows_lds_bytes<FP4_FMT_NVFP4>() : kBatchLds];
  const uint32_t b = blockIdx.x;
  uint32_t s = 0;
  for (uint32_t i = 1; i < A.nseg; ++i) s = b >= A.first[i] ? i : s;
  const BatchSeg& S = A.seg[s];
  const uint32_t bid = b - A.first[s];
  constexpr int AB = FP4_SCALE_ABSMAX;
  if constexpr (NV_ROWS) {
#define FP4_SEG_NV(F, R)                                                                       \
  case seg_sel(kSegRows, F, R):                                                                \
    quant_rows_body<F, R, 2, AB, 0>(lds, bid, S.nwg, S.x, S.ldx_bytes, S.rows, S.nb, S.aux,    \
                                    S.codes, S.scales, S.kchunks, 0, S.gs, S.partials,         \
                                    S.npart, S.P);                                             \
    break;
    switch (S.sel) {
      FP4_SEG_NV(FP4_FMT_NVFP4, 0)
      FP4_SEG_NV(FP4_FMT_NVFP4, 1)
      FP4_SEG_NV(FP4_FMT_NVINT4, 0)
      FP4_SEG_NV(FP4_FMT_NVINT4, 1)
      default:
        break;
    }
#undef FP4_SEG_NV
    return;
  }
  switch (S.sel) {
#define FP4_SEG_MXG(F, R)                                                                      \
  case seg_sel(kSegMxGemm, F, R):                                                              \
    quant_mx_gemm_body<F, R, AB, 0>(lds, bid, S.nwg, S.x, S.ldx_bytes, S.rows, S.nb, S.aux,    \
                                    S.codes, S.scales, S.kchunks, S.P);                        \
    break;
#define FP4_SEG_ROWS(F, R)                                                                     \
  case seg_sel(kSegRows, F, R):                                                                \
    quant_rows_body<F, R, fmt_mx(F) ? 1 : 2, AB, 0>(lds, bid, S.nwg, S.x, S.ldx_bytes, S.rows, \
                                                    S.nb, S.aux, S.codes, S.scales, S.kchunks, \
                                                    0, S.gs, S.partials, S.npart, S.P);        \
    break;
    FP4_SEG_MXG(FP4_FMT_MXFP4, 0)
    FP4_SEG_MXG(FP4_FMT_MXFP4, 1)
    FP4_SEG_MXG(FP4_FMT_MXINT4, 0)
    FP4_SEG_MXG(FP4_FMT_MXINT4, 1)
    FP4_SEG_ROWS(FP4_FMT_MXFP4, 0)
    FP4_SEG_ROWS(FP4_FMT_MXINT4, 0)
    FP4_SEG_ROWS(FP4_FMT_MXFP4, 1)
    FP4_SEG_ROWS(FP4_FMT_MXINT4, 1)
    FP4_SEG_ROWS(FP4_FMT_NVFP4, 0)
    FP4_SEG_ROWS(FP4_FMT_NVFP4, 1)
    FP4_SEG_ROWS(FP4_FMT_NVINT4, 0)
    FP4_SEG_ROWS(FP4_FMT_NVINT4, 1)
#undef FP4_SEG_ROWS
#undef FP4_SEG_MXG
    case seg_sel(kSegAmax, 0, 0):
      amax_chunk_body<false, kThreads / 64>(reinterpret_cast<float*>(lds), bid, S.nwg, S.x,
                                            S.ldx_bytes, S.rows, S.aux, S.aux2, S.partials, 0u);
      break;
    case seg_sel(kSegAmax, 0, 1):
      amax_chunk_body<true, kThreads / 64>(reinterpret_cast<float*>(lds), bid, S.nwg, S.x,
                                           S.ldx_bytes, S.rows, S.aux, S.aux2, S.partials,
                                           S.P.signs[0]);
      break;
    default:
      break;
  }
}

// ---------------------------------------------------------- direct kernel
// Any shape: each thread loads its own block.
template <int FMT, int XDT, int ROT, int RULE, int RND>
__global__ __launch_bounds__(kThreads) void quant_direct_kernel(
    const void* __restrict__ x, int64_t ldx, uint32_t rows, uint32_t nb,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t kchunks, int gemm_layout,
    float* __restrict__ gs, const float* __restrict__ partials, int npart, QParams P) {
  constexpr int G = fmt_block(FMT);
  constexpr int ES = XDT == FP4_DT_BF16 ? 2 : 4;
  constexpr int CH = G * ES / 16;
  NvTs T{};
  if constexpr (!fmt_mx(FMT)) T = nv_launch_ts<FMT>(gs, partials, npart);
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) +
                                                    ((int64_t)r * ldx + (int64_t)kb * G) * ES);
    u32x4 c[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) c[k] = p[k];
    quantize_block<FMT, XDT, ROT, RULE, RND>(c, T, r, kb, nb, codes, scales, kchunks, gemm_layout, P);
  }
}

// --------------------------------------------------------------- amax pass
// Plain tensor: the maximum |x| needs no block structure, so every 16-byte
// chunk of every row is read once, fully coalesced.  One partial per workgroup.
template <int XDT>
__global__ __launch_bounds__(kThreads) void amax_plain_kernel(const void* __restrict__ x,
                                                              int64_t ldx, uint32_t rows,
                                                              uint32_t cpr,
                                                              float* __restrict__ partials) {
  constexpr int ES = XDT == FP4_DT_BF16 ? 2 : 4;
  const uint32_t total = rows * cpr;  // 16-byte chunks
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t mb = 0;  // bf16: max of |x| bits (15 bits)
  float mf = 0.0f;
  for (uint32_t i0 = blockIdx.x * kThreads + threadIdx.x; i0 < total; i0 += 4 * stride) {
    u32x4 t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + u * stride;
      if (i < total) {
        const uint32_t r = i / cpr, c = i - r * cpr;
        t[u] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) + (int64_t)r * ldx * ES + (int64_t)c * 16);
      } else {
        t[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (XDT == FP4_DT_BF16) {
        u16x2 m = {0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, t[u][j] & 0x7FFF7FFFu));
        mb = max(mb, (uint32_t)max(m[0], m[1]));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) mf = fmaxf(mf, fabsf(as_f(t[u][j])));
      }
    }
  }
  float m = XDT == FP4_DT_BF16 ? as_f(mb << 16) : mf;
  m = wg_max(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Rotated tensor: the maximum of the block-Hadamard outputs, block by block.
template <int XDT>
__global__ __launch_bounds__(kThreads) void amax_rot_kernel(const void* __restrict__ x, int64_t ldx,
                                                            uint32_t rows, uint32_t nb,
                                                            float* __restrict__ partials,
                                                            uint32_t sign_mask) {
  constexpr int ES = XDT == FP4_DT_BF16 ? 2 : 4;
  constexpr int CH = 16 * ES / 16;
  float m = 0.0f;
  const uint32_t total = rows * nb;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t r = b / nb;
    const uint32_t kb = b - r * nb;
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) +
                                                    ((int64_t)r * ldx + (int64_t)kb * 16) * ES);
    u32x4 c[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) c[k] = p[k];
    float v[16];
    unpack<XDT, 16>(c, v);
    if (sign_mask) apply_signs<16>(v, sign_mask);
    fwht<16>(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = wg_max(m) * 0.25f;  // 1/sqrt(16), exact
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Reduce the partial maxima into ts = amax / tdiv (one workgroup; tdiv =
// 448 * qmax of the element).
__global__ __launch_bounds__(kThreads) void amax_final_kernel(const float* __restrict__ partials,
                                                              int npart, float* __restrict__ gs,
                                                              float tdiv) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < npart; i += kThreads) m = fmaxf(m, partials[i]);
  m = wg_max(m);
  if (threadIdx.x == 0) *gs = m / tdiv;
}

__global__ void set_scalar_kernel(float* p, float v) { *p = v; }

// Zero n dwords (a workspace; a kernel rather than a memset so that it can sit
// in a captured graph).
__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0u;
}

// Row-major [rows, nb] MXFP4 scales -> GEMM layout (padding filled with 127).
__global__ __launch_bounds__(kThreads) void scales_to_gemm_kernel(const uint8_t* __restrict__ src,
                                                                  uint32_t rows, uint32_t nb,
                                                                  uint32_t kchunks,
                                                                  uint8_t* __restrict__ dst,
                                                                  uint32_t total) {
  for (uint32_t p = blockIdx.x * kThreads + threadIdx.x; p < total; p += gridDim.x * kThreads) {
    const uint32_t tile = p >> 8, within = p & 255u;
    const uint32_t dw = within >> 2, j = within & 3u;
    const uint32_t h = dw >> 5, rr = dw & 31u;
    const uint32_t rt = tile / kchunks, kc = tile - rt * kchunks;
    const uint32_t r = rt * 32 + rr, kb = kc * 8 + 2 * j + h;
    dst[p] = (r < rows && kb < nb) ? src[(int64_t)r * nb + kb] : (uint8_t)127;
  }
}

int grid_cap(int64_t items, int cap) {
  int64_t g = (items + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

template <int FMT, int XDT, int ROT, int RULE, int RND>
hipError_t launch_q(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, int gemm_layout, float* gs, const float* partials, int npart,
                    const QParams& P, hipStream_t st) {
  constexpr int G = fmt_block(FMT);
  const uint32_t nb = (uint32_t)(cols / G);
  const int64_t kchunks = mx_gemm_kchunks(cols);
  if constexpr (XDT == FP4_DT_BF16) {
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    if constexpr (fmt_mx(FMT)) {
      if (gemm_layout) {
        const uint32_t kcs = (nb + 7) / 8;
        int64_t g = ((rows + 31) / 32) * (int64_t)kcs;
        if (g > 16384) g = 16384;
        quant_mx_gemm_kernel<FMT, ROT, RULE, RND><<<(int)g, kThreads, 0, st>>>(
            xb, ldx * 2, (uint32_t)rows, nb, kcs, codes, scales, kchunks, P);
        return hipGetLastError();
      }
    }
    constexpr int TPW = fmt_mx(FMT) ? 1 : 2;
    const uint32_t wpr = (nb + 63) / 64;
    const int64_t waves = (rows * (int64_t)wpr + TPW - 1) / TPW;
    int64_t g = (waves + kThreads / 64 - 1) / (kThreads / 64);
    if (g > 8192) g = 8192;
    quant_rows_kernel<FMT, ROT, TPW, RULE, RND><<<(int)g, kThreads, 0, st>>>(
        xb, ldx * 2, (uint32_t)rows, nb, wpr, codes, scales, kchunks, gemm_layout, gs, partials,
        npart, P);
    return hipGetLastError();
  }
  if (nb % 64 == 0) {
    const int64_t waves = rows * (int64_t)(nb / 64);
    int64_t g = (waves + 3) / 4;
    if (g > 4096) g = 4096;
    quant_tile_kernel<FMT, XDT, ROT, RULE, RND><<<(int)g, kThreads, 0, st>>>(
        x, ldx, (uint32_t)rows, nb, codes, scales, kchunks, gemm_layout, gs, partials, npart, P);
  } else {
    quant_direct_kernel<FMT, XDT, ROT, RULE, RND><<<grid_cap(rows * (int64_t)nb, 8192), kThreads, 0, st>>>(
        x, ldx, (uint32_t)rows, nb, codes, scales, kchunks, gemm_layout, gs, partials, npart, P);
  }
  return hipGetLastError();
}

// -------------------------------------------------- NVFP4 16x16 weight blocks
// One scale per tile of 16 rows x one 16-column block, stored for each of
// its rows ("NVFP4 vs MXFP4 ...", two-dimensional weight scaling: a tile and
// its transpose share the scale).  Wave tile = 16 rows x 64 blocks; lane l
// owns block 64 w + l of the 16 rows: a first sweep over the rows takes the
// tile maximum, a second re-reads each row (from cache), encodes and stores.
// Each lane loads its own 32 bytes (bf16) or 64 bytes (fp32) per row, so a
// wave reads 2 or 4 KB of one row contiguously.
template <int XDT, int RND>
__global__ __launch_bounds__(kThreads) void quant_nv2d_kernel(
    const void* __restrict__ x, int64_t ldx, uint32_t rows, uint32_t nb, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gs, const float* __restrict__ partials,
    int npart, QParams P) {
  constexpr int ES = XDT == FP4_DT_BF16 ? 2 : 4;
  constexpr int CH = 16 * ES / 16;  // 16-byte chunks per block
  const NvTs T = nv_launch_ts<FP4_FMT_NVFP4>(gs, partials, npart);
  const int lane = threadIdx.x & 63;
  const uint32_t wpr = (nb + 63) / 64, rts = (rows + 15) / 16;
  const uint32_t tiles = rts * wpr;
  for (uint32_t tile = blockIdx.x * (kThreads / 64) + wave_index(); tile < tiles;
       tile += gridDim.x * (kThreads / 64)) {
    const uint32_t rt = tile / wpr, w = tile - rt * wpr;
    const uint32_t kb = w * 64 + lane;
    if (kb >= nb) continue;
    const uint32_t r0 = rt * 16, r1 = min(r0 + 16, rows);
    auto load = [&](uint32_t r, float* v) __attribute__((always_inline)) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) +
                                                      ((int64_t)r * ldx + (int64_t)kb * 16) * ES);
      u32x4 c[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) c[k] = p[k];
      unpack<XDT, 16>(c, v);
    };
    float amax = 0.0f;
    for (uint32_t r = r0; r < r1; ++r) {
      float v[16];
      load(r, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    float s;
    const uint32_t code = nv_scale(amax, T, s);
    for (uint32_t r = r0; r < r1; ++r) {
      float v[16];
      load(r, v);
      u32x2 o;
      if constexpr (RND != 0) {
        if (s == 0.0f) {
          o = u32x2{0u, 0u};
        } else {
          if (s >= 0x1p-100f) {
            const float rs = 1.0f / s;
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = div_rn(v[i], s, rs);
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v[i] / s;
          }
          uint32_t wds[16];
          sr_words<16>((uint64_t)r * (uint64_t)P.cols + (uint64_t)kb * 16, P, wds);
          o = u32x2{enc8_sr(&v[0], &wds[0]), enc8_sr(&v[8], &wds[8])};
        }
      } else {
        o = u32x2{nv_enc8(&v[0], s), nv_enc8(&v[8], s)};
      }
      *reinterpret_cast<u32x2*>(codes + code_offset(r, (int64_t)kb * 8, (int64_t)nb * 8, P.tiled != 0)) = o;
      scales[(int64_t)r * nb + kb] = (uint8_t)code;
    }
  }
}

}  // namespace

namespace fp4lib {

int amax_partials(int64_t rows, int64_t cols, int rotate, int xdt) {
  // one partial per workgroup of the amax pass
  if (xdt == FP4_DT_BF16) {
    const int64_t tiles = rows * ((cols / 8 + 255) / 256);
    int64_t g = (tiles + kAmaxThreads / 64 - 1) / (kAmaxThreads / 64);
    if (g > kAmaxGrid) g = kAmaxGrid;
    return (int)(g < 1 ? 1 : g);
  }
  const int64_t items = rotate ? rows * (cols / 16) : rows * ((cols + 7) / 8);
  return grid_cap(items / 4 + 1, kAmaxGrid);
}

// Instantiate launch_q for one format over input type x rotation size.
template <int FMT, int RULE, int RND>
hipError_t launch_q_rule(const void* x, int xdt, int rot_blocks, int64_t rows, int64_t cols,
                         int64_t ldx, uint8_t* codes, uint8_t* scales, int gemm_layout, float* gs,
                         const float* partials, int npart, const QParams& P, hipStream_t st) {
#define FP4_LQ(X, R)                                                                              \
  return launch_q<FMT, X, R, RULE, RND>(x, rows, cols, ldx, codes, scales, gemm_layout, gs,        \
                                        partials, npart, P, st)
#define FP4_LQ_X(R)                           \
  do {                                        \
    if (xdt == FP4_DT_BF16) FP4_LQ(FP4_DT_BF16, R); \
    FP4_LQ(FP4_DT_F32, R);                    \
  } while (0)
  if (rot_blocks == 0) FP4_LQ_X(0);
  if constexpr (fmt_mx(FMT)) {
    if (rot_blocks == 2) FP4_LQ_X(2);
    if (rot_blocks == 4) FP4_LQ_X(4);
  }
  FP4_LQ_X(1);
#undef FP4_LQ_X
#undef FP4_LQ
}

hipError_t launch_quantize_mx(int fmt, const void* x, int xdt, int rot_blocks, int rule,
                              int rounding, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                              uint8_t* scales, int gemm_layout, const QParams& P, hipStream_t st) {
  if (fmt == FP4_FMT_MXINT4)
    return launch_q_rule<FP4_FMT_MXINT4, FP4_SCALE_ABSMAX, 0>(x, xdt, rot_blocks, rows, cols, ldx, codes, scales, gemm_layout, nullptr, nullptr, 0, P, st);
  if (rounding != 0)
    return launch_q_rule<FP4_FMT_MXFP4, FP4_SCALE_ABSMAX, 1>(x, xdt, rot_blocks, rows, cols, ldx, codes, scales, gemm_layout, nullptr, nullptr, 0, P, st);
  if (rule == FP4_SCALE_MSE)
    return launch_q_rule<FP4_FMT_MXFP4, FP4_SCALE_MSE, 0>(x, xdt, rot_blocks, rows, cols, ldx, codes, scales, gemm_layout, nullptr, nullptr, 0, P, st);
  return launch_q_rule<FP4_FMT_MXFP4, FP4_SCALE_ABSMAX, 0>(x, xdt, rot_blocks, rows, cols, ldx, codes, scales, gemm_layout, nullptr, nullptr, 0, P, st);
}

hipError_t launch_amax_nv(const void* x, int xdt, int rotate, uint32_t sign_mask, int64_t rows,
                          int64_t cols, int64_t ldx, float* partials, int npart, hipStream_t st) {
  const int es = xdt == FP4_DT_BF16 ? 2 : 4;
  if (xdt == FP4_DT_BF16) {
    const uint32_t cpr = (uint32_t)(cols / 8);
    const uint32_t wpr = (cpr + 255) / 256;
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    if (rotate)
      amax_chunk_kernel<true><<<npart, kAmaxThreads, 0, st>>>(xb, ldx * 2, (uint32_t)rows, cpr, wpr, partials, sign_mask);
    else
      amax_chunk_kernel<false><<<npart, kAmaxThreads, 0, st>>>(xb, ldx * 2, (uint32_t)rows, cpr, wpr, partials, 0u);
    return hipGetLastError();
  }
  if (rotate) {
    if (xdt == FP4_DT_BF16)
      amax_rot_kernel<FP4_DT_BF16><<<npart, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, (uint32_t)(cols / 16), partials, sign_mask);
    else
      amax_rot_kernel<FP4_DT_F32><<<npart, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, (uint32_t)(cols / 16), partials, sign_mask);
  } else {
    const uint32_t cpr = (uint32_t)(cols * es / 16);
    if (xdt == FP4_DT_BF16)
      amax_plain_kernel<FP4_DT_BF16><<<npart, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, cpr, partials);
    else
      amax_plain_kernel<FP4_DT_F32><<<npart, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, cpr, partials);
  }
  return hipGetLastError();
}

hipError_t launch_amax_final(int fmt, const float* partials, int npart, float* gs, hipStream_t st) {
  if (npart <= 0) {
    set_scalar_kernel<<<1, 1, 0, st>>>(gs, 0.0f);
  } else {
    amax_final_kernel<<<1, kThreads, 0, st>>>(partials, npart, gs, 448.0f * fmt_qmax(fmt));
  }
  return hipGetLastError();
}

// CU count of the current device (queried once per device); 0 on failure.
int device_cus() {
  static std::atomic<int> cus_of[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cus = cus_of[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

template <int FMT, int ROT, int RULE, int RND>
hipError_t fused_launch(int tpw, const uint8_t* x, int64_t rows, int64_t ldx_bytes, uint32_t nb,
                        uint32_t wpr, uint8_t* codes, uint8_t* scales, float* gs, uint32_t* xchg,
                        const QParams& P, hipStream_t st) {
  const int64_t tiles = rows * (int64_t)wpr;
  const int64_t grid = (tiles + (int64_t)kFusedWaves * tpw - 1) / ((int64_t)kFusedWaves * tpw);
  if (tpw == 4)
    quant_nv_fused_kernel<FMT, ROT, 4, RULE, RND><<<(unsigned)grid, kFusedThreads, 0, st>>>(
        x, ldx_bytes, (uint32_t)rows, nb, wpr, codes, scales, gs, xchg, P);
  else
    quant_nv_fused_kernel<FMT, ROT, 8, RULE, RND><<<(unsigned)grid, kFusedThreads, 0, st>>>(
        x, ldx_bytes, (uint32_t)rows, nb, wpr, codes, scales, gs, xchg, P);
  return hipGetLastError();
}

template <int FMT, int RULE, int RND>
hipError_t fused_rule(int tpw, const uint8_t* x, int rotate, int64_t rows, int64_t ldx_bytes,
                      uint32_t nb, uint32_t wpr, uint8_t* codes, uint8_t* scales, float* gs,
                      uint32_t* xchg, const QParams& P, hipStream_t st) {
  if (rotate)
    return fused_launch<FMT, 1, RULE, RND>(tpw, x, rows, ldx_bytes, nb, wpr, codes, scales, gs, xchg, P, st);
  return fused_launch<FMT, 0, RULE, RND>(tpw, x, rows, ldx_bytes, nb, wpr, codes, scales, gs, xchg, P, st);
}

int quantize_nv_one_pass_tpw(int xdt, int block_rows, int64_t rows, int64_t cols, int64_t ldx,
                             int max_grid) {
  if (xdt != FP4_DT_BF16 || block_rows == 16 || rows <= 0 || cols <= 0 || (ldx * 2) % 16 != 0)
    return 0;
  const int cus = device_cus();
  const int64_t cap = cus < max_grid ? cus : max_grid;  // one workgroup per CU
  const int64_t tiles = rows * ((cols / 16 + 63) / 64);
  for (int tpw = 4; tpw <= 8; tpw *= 2)
    if ((tiles + (int64_t)kFusedWaves * tpw - 1) / ((int64_t)kFusedWaves * tpw) <= cap) return tpw;
  return 0;
}

hipError_t launch_quantize_nv_one_pass(int fmt, const void* x, int xdt, int rotate, int rule,
                                       int rounding, int block_rows, int64_t rows, int64_t cols,
                                       int64_t ldx, uint8_t* codes, uint8_t* scales, float* gs,
                                       uint32_t* xchg, int max_grid, const QParams& P,
                                       hipStream_t st) {
  const int tpw = quantize_nv_one_pass_tpw(xdt, block_rows, rows, cols, ldx, max_grid);
  if (tpw == 0) return hipErrorNotSupported;
  const uint32_t nb = (uint32_t)(cols / 16), wpr = (nb + 63) / 64;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const int64_t lb = ldx * 2;
  if (fmt == FP4_FMT_NVINT4)
    return fused_rule<FP4_FMT_NVINT4, FP4_SCALE_ABSMAX, 0>(tpw, xb, rotate, rows, lb, nb, wpr, codes, scales, gs, xchg, P, st);
  if (rounding != 0)
    return fused_rule<FP4_FMT_NVFP4, FP4_SCALE_ABSMAX, 1>(tpw, xb, rotate, rows, lb, nb, wpr, codes, scales, gs, xchg, P, st);
  if (rule == FP4_SCALE_MSE)
    return fused_rule<FP4_FMT_NVFP4, FP4_SCALE_MSE, 0>(tpw, xb, rotate, rows, lb, nb, wpr, codes, scales, gs, xchg, P, st);
  if (rule == FP4_SCALE_FOUR_OVER_SIX)
    return fused_rule<FP4_FMT_NVFP4, FP4_SCALE_FOUR_OVER_SIX, 0>(tpw, xb, rotate, rows, lb, nb, wpr, codes, scales, gs, xchg, P, st);
  return fused_rule<FP4_FMT_NVFP4, FP4_SCALE_ABSMAX, 0>(tpw, xb, rotate, rows, lb, nb, wpr, codes, scales, gs, xchg, P, st);
}

hipError_t launch_quantize_nv(int fmt, const void* x, int xdt, int rotate, int rule, int rounding,
                              int block_rows, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* gs, const float* partials,
                              int npart, const QParams& P, hipStream_t st) {
  if (block_rows == 16) {
    const uint32_t nb = (uint32_t)(cols / 16);
    const int64_t tiles = ((rows + 15) / 16) * (int64_t)((nb + 63) / 64);
    int64_t g = (tiles + 3) / 4;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
#define FP4_2D(X, R) \
    quant_nv2d_kernel<X, R><<<(int)g, kThreads, 0, st>>>(x, ldx, (uint32_t)rows, nb, codes, scales, gs, partials, npart, P)
    if (xdt == FP4_DT_BF16) {
      if (rounding) FP4_2D(FP4_DT_BF16, 1); else FP4_2D(FP4_DT_BF16, 0);
    } else {
      if (rounding) FP4_2D(FP4_DT_F32, 1); else FP4_2D(FP4_DT_F32, 0);
    }
#undef FP4_2D
    return hipGetLastError();
  }
  const int rb = rotate ? 1 : 0;
  if (fmt == FP4_FMT_NVINT4)
    return launch_q_rule<FP4_FMT_NVINT4, FP4_SCALE_ABSMAX, 0>(x, xdt, rb, rows, cols, ldx, codes, scales, 0, gs, partials, npart, P, st);
  if (rounding != 0)
    return launch_q_rule<FP4_FMT_NVFP4, FP4_SCALE_ABSMAX, 1>(x, xdt, rb, rows, cols, ldx, codes, scales, 0, gs, partials, npart, P, st);
  if (rule == FP4_SCALE_MSE)
    return launch_q_rule<FP4_FMT_NVFP4, FP4_SCALE_MSE, 0>(x, xdt, rb, rows, cols, ldx, codes, scales, 0, gs, partials, npart, P, st);
  if (rule == FP4_SCALE_FOUR_OVER_SIX)
    return launch_q_rule<FP4_FMT_NVFP4, FP4_SCALE_FOUR_OVER_SIX, 0>(x, xdt, rb, rows, cols, ldx, codes, scales, 0, gs, partials, npart, P, st);
  return launch_q_rule<FP4_FMT_NVFP4, FP4_SCALE_ABSMAX, 0>(x, xdt, rb, rows, cols, ldx, codes, scales, 0, gs, partials, npart, P, st);
}

int batch_amax_partials(int64_t rows, int64_t cols) {
  const int64_t tiles = rows * ((cols / 8 + 255) / 256);
  int64_t g = (tiles + kThreads / 64 - 1) / (kThreads / 64);
  if (g > kAmaxGrid) g = kAmaxGrid;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_quantize_batch(const BatchItem* items, int n, hipStream_t st) {
  BatchArgs A{};
  uint32_t wgs = 0;
  bool nv_rows_only = false;  // the second launch
  hipError_t err = hipSuccess;
  auto flush = [&]() {
    if (A.nseg > 0 && err == hipSuccess) {
      if (nv_rows_only)
        quant_batch_kernel<true><<<wgs, kThreads, 0, st>>>(A);
      else
        quant_batch_kernel<false><<<wgs, kThreads, 0, st>>>(A);
      err = hipGetLastError();
    }
    A.nseg = 0;
    wgs = 0;
  };
  auto add = [&](const BatchSeg& seg) {
    if (A.nseg == (uint32_t)kBatchSegs) flush();
    A.seg[A.nseg] = seg;
    A.first[A.nseg] = wgs;
    wgs += seg.nwg;
    ++A.nseg;
  };
  auto base = [](const BatchItem& it) {
    BatchSeg g{};
    g.x = static_cast<const uint8_t*>(it.x);
    g.codes = it.codes;
    g.scales = it.scales;
    g.gs = it.gs;
    g.ldx_bytes = it.ldx * 2;
    g.kchunks = mx_gemm_kchunks(it.cols);
    g.rows = (uint32_t)it.rows;
    g.nb = (uint32_t)(it.cols / fmt_block(it.fmt));
    g.P = it.P;
    return g;
  };
  auto encode_seg = [&](const BatchItem& it, int npart) {
    BatchSeg g = base(it);
    const int rot = it.rotate ? 1 : 0;
    if (fmt_mx(it.fmt) && it.gemm_layout) {
      const uint32_t kcs = (g.nb + 7) / 8;
      int64_t wg = ((it.rows + 31) / 32) * (int64_t)kcs;
      g.nwg = (uint32_t)(wg > 16384 ? 16384 : wg);
      g.aux = kcs;
      g.sel = seg_sel(kSegMxGemm, it.fmt, rot);
    } else {
      const int tpw = fmt_mx(it.fmt) ? 1 : 2;
      const uint32_t wpr = (g.nb + 63) / 64;
      const int64_t waves = (it.rows * (int64_t)wpr + tpw - 1) / tpw;
      int64_t wg = (waves + kThreads / 64 - 1) / (kThreads / 64);
      g.nwg = (uint32_t)(wg > 8192 ? 8192 : wg);
      g.aux = wpr;
      g.partials = it.partials;
      g.npart = npart;
      g.sel = seg_sel(kSegRows, it.fmt, rot);
    }
    add(g);
  };
  // launch 1: the maxima first (their workgroups run longest), then every
  // encoding that needs nothing else
  for (int i = 0; i < n; ++i) {
    const BatchItem& it = items[i];
    if (it.partials == nullptr) continue;
    BatchSeg g = base(it);
    g.nwg = (uint32_t)batch_amax_partials(it.rows, it.cols);
    g.aux = (uint32_t)(it.cols / 8);
    g.aux2 = (g.aux + 255) / 256;
    g.partials = it.partials;
    g.sel = seg_sel(kSegAmax, 0, it.rotate ? 1 : 0);
    add(g);
  }
  for (int i = 0; i < n; ++i)
    if (items[i].partials == nullptr) encode_seg(items[i], 0);
  flush();
  // launch 2: the encodings that read the maxima of launch 1
  nv_rows_only = true;
  for (int i = 0; i < n; ++i)
    if (items[i].partials != nullptr) encode_seg(items[i], batch_amax_partials(items[i].rows, items[i].cols));
  flush();
  return err;
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  zero_words_kernel<<<grid_cap(n, 64), kThreads, 0, st>>>(p, (uint32_t)n);
  return hipGetLastError();
}

hipError_t launch_scales_to_gemm(const uint8_t* src, int64_t rows, int64_t cols, uint8_t* dst,
                                 hipStream_t st) {
  const uint32_t nb = (uint32_t)(cols / 32);
  const int64_t kchunks = mx_gemm_kchunks(cols);
  const int64_t total = ((rows + 31) / 32) * kchunks * 256;
  if (total == 0) return hipSuccess;
  scales_to_gemm_kernel<<<grid_cap(total, 8192), kThreads, 0, st>>>(src, (uint32_t)rows, nb,
                                                                    (uint32_t)kchunks, dst,
                                                                    (uint32_t)total);
  return hipGetLastError();
}

}  // namespace fp4lib
