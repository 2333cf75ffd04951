// gemm.hip -- FP4 x FP4 block-scaled GEMMs for gfx950, Y = A * B^T with fp32
// accumulation ("Bridging the Gap Between Promise and Performance for
// Microscaling FP4 Quantization": the kernels compute Q(W H_k) Q(X H_k)^T;
// "NVFP4 vs MXFP4: 4-Bit Floating Point for LLM Training and Inference
// (2026)", hardware execution: scales applied inside the product, higher
// precision accumulation).
//
// MXFP4 runs on the CDNA4 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// E2M1 operands): E8M0 scales are fed per 32-K block straight from the
// GEMM scale layout, one dword per lane holding four consecutive 64-K steps
// (selected with the instruction's byte select).
//
// NVFP4 has no E4M3-scaled MFMA: each K-tile is dequantized into LDS as fp16,
// e2m1 * e4m3 being exact in fp16 (at most 6 significant bits, magnitudes in
// [2^-10, 2688]), and multiplied on the fp16 MFMA; the fp32 tensor scales
// multiply the accumulator in the epilogue ("Portable FP4 Quantization for
// Heterogeneous Accelerators", section 2.5: conversion fused with GEMM entry
// instead of materialising a full-precision copy).
#include "fp4_device.h"
#include "launch.h"

using namespace fp4k;

namespace {

constexpr int kThreads = 256;

// XOR swizzle of 16-byte chunks within a 64-byte LDS row (4 chunks): rows 2r
// and 2r+1 fall on different banks and 8 (or 16) consecutive rows read by one
// ds_read_b128 group hit distinct banks.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
// Same for 128-byte rows (8 chunks).
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

template <int YDT>
__device__ __forceinline__ void store_out(void* __restrict__ Y, int64_t ldy, int row, int col,
                                          float v) {
  if constexpr (YDT == FP4_DT_F32) {
    static_cast<float*>(Y)[(int64_t)row * ldy + col] = v;
  } else {
    static_cast<uint16_t*>(Y)[(int64_t)row * ldy + col] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// ------------------------------------------------------------------ MXFP4
// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs (each with its own L2); consecutive ids are first regrouped per XCD,
// then walked in groups of GROUP_M tile rows so that the workgroups running on
// one XCD share a compact block of A and B tiles.
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Block tile BM x BN, K-stage of 128 (64 bytes of codes per row), waves each
// owning a WM x WN sub-tile made of 32x32 MFMA tiles.  Software pipeline:
// global loads run two stages ahead through two register sets, LDS is double
// buffered, and the scale dwords (one per 256-K chunk, four MFMA steps) run
// one chunk ahead.  With PARTIAL, blockIdx.y selects a K-slice (an even number
// of stages) and fp32 partial sums go to the workspace.
template <int BM, int BN, int WM, int WN, int YDT, bool PARTIAL>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN)) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, void* __restrict__ Y, int64_t ldy, int M, int N, int K,
    int kchunks, int tiles_n, int kt_per_split, float* __restrict__ part) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NT = 64 * (BM / WM) * (BN / WN);  // threads per workgroup
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CHUNKS = BM * 4, B_CHUNKS = BN * 4;  // 16-byte chunks per stage
  constexpr int A_PER = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER = (B_CHUNKS + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // per-thread source rows (clamped into the matrix) and chunk columns
  const uint8_t* a_src[A_PER];
  const uint8_t* b_src[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int c = tid + i * NT;
    a_src[i] = A + (int64_t)min(m0 + (c >> 2), M - 1) * rowbytes + (c & 3) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int c = tid + i * NT;
    b_src[i] = B + (int64_t)min(n0 + (c >> 2), N - 1) * rowbytes + (c & 3) * 16;
  }

  u32x4 ra[2][A_PER], rb[2][B_PER];
  auto gload = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      if (A_CHUNKS % NT == 0 || tid + i * NT < A_CHUNKS)
        ra[slot][i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * 64);
#pragma unroll
    for (int i = 0; i < B_PER; ++i)
      if (B_CHUNKS % NT == 0 || tid + i * NT < B_CHUNKS)
        rb[slot][i] = *reinterpret_cast<const u32x4*>(b_src[i] + kt * 64);
  };
  auto lstore = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      if (A_CHUNKS % NT == 0 || c < A_CHUNKS) {
        const int row = c >> 2;
        *reinterpret_cast<u32x4*>(&lds[buf][row * 64 + (((c & 3) ^ swz4(row)) * 16)]) = ra[slot][i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      if (B_CHUNKS % NT == 0 || c < B_CHUNKS) {
        const int row = c >> 2;
        *reinterpret_cast<u32x4*>(&lds[buf][BM * 64 + row * 64 + (((c & 3) ^ swz4(row)) * 16)]) = rb[slot][i];
      }
    }
  };
  // Scale dwords of this wave's 32-row tiles for 256-K chunk kc.
  const uint8_t* as_src[TM];
  const uint8_t* bs_src[TN];
  const int rt_max = (M - 1) >> 5, ct_max = (N - 1) >> 5;
#pragma unroll
  for (int i = 0; i < TM; ++i)
    as_src[i] = As + (int64_t)min((m0 + wm * WM + i * 32) >> 5, rt_max) * kchunks * 256 + lane * 4;
#pragma unroll
  for (int j = 0; j < TN; ++j)
    bs_src[j] = Bs + (int64_t)min((n0 + wn * WN + j * 32) >> 5, ct_max) * kchunks * 256 + lane * 4;
  uint32_t sa_cur[TM], sb_cur[TN], sa_nxt[TM], sb_nxt[TN];
  auto sload = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_nxt[i] = *reinterpret_cast<const uint32_t*>(as_src[i] + kc * 256);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_nxt[j] = *reinterpret_cast<const uint32_t*>(bs_src[j] + kc * 256);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // two MFMA K-steps (sel = first scale byte) from LDS buffer buf
  auto compute = [&](int buf, int sel0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8 af[TM], bf[TN];
      const int q = s * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        const u32x4 t = *reinterpret_cast<const u32x4*>(&lds[buf][row * 64 + ((q ^ swz4(row)) * 16)]);
        af[i] = i32x8{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        const u32x4 t = *reinterpret_cast<const u32x4*>(&lds[buf][BM * 64 + row * 64 + ((q ^ swz4(row)) * 16)]);
        bf[j] = i32x8{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
      }
      const int sh = 8 * (sel0 + s);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], 4, 4, 0, (int)(sa_cur[i] >> sh), 0, (int)(sb_cur[j] >> sh));
    }
  };

  if (kt0 < kt1) {
    sload(kt0 >> 1);
    gload(kt0, 0);
    if (kt0 + 1 < kt1) gload(kt0 + 1, 1);
    lstore(0, 0);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; kt += 2) {
    // even stage kt: LDS buffer 0, scale bytes 0 and 1 of chunk kt/2
#pragma unroll
    for (int i = 0; i < TM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb_cur[j] = sb_nxt[j];
    if (kt + 2 < kt1) {
      sload((kt >> 1) + 1);
      gload(kt + 2, 0);
    }
    compute(0, 0);
    if (kt + 1 < kt1) lstore(1, 1);
    __syncthreads();
    if (kt + 1 >= kt1) break;
    // odd stage kt+1: LDS buffer 1, scale bytes 2 and 3
    if (kt + 3 < kt1) gload(kt + 3, 1);
    compute(1, 2);
    if (kt + 2 < kt1) lstore(0, 0);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (row < M && col < N) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e]);
        }
      }
}

// Large-tile MXFP4 kernel: 256 x 256 block tile, four waves of 128 x 128
// (4 x 4 MFMA tiles, accumulators in AGPRs).  Codes and scale tiles stream
// straight from global memory into a 4-slot LDS ring
// (global_load_lds_dwordx4, no staging registers) three 128-K stages ahead of
// the MFMAs.  Each lane picks the source chunk that belongs at its LDS
// position, which applies the XOR swizzle.  A slot holds the stage's A and B
// codes (2 x 16 KB) and the 16 scale tiles of its 256-K chunk (4 KB): nine
// 16-byte DMAs per thread per stage and no other global loads in the loop, so
// one exact wait (vmcnt = the two later stages' 18 loads) and one barrier per
// stage suffice.  Stages past the end re-load the last stage into the slot
// that is free, keeping the count constant.
constexpr int kDmaStages = 4;
constexpr int kDmaCodeBytes = (256 + 256) * 64;
constexpr int kDmaStageBytes = kDmaCodeBytes + 16 * 256;

template <int YDT, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_mx_dma_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, void* __restrict__ Y, int64_t ldy, int M, int N, int K,
    int kchunks, int tiles_n, int kt_per_split, float* __restrict__ part) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, TM = 4, TN = 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  typedef __attribute__((address_space(3))) void* lds_ptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // Code DMAs: instruction i (0..7) of this thread fills slot bytes
  // [(i*4 + wave)*1024 + lane*16, +16), i.e. row (i*4 + wave)*16 + lane/4
  // (A rows 0..255, then B rows), chunk lane%4.
  const uint8_t* src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (i * 4 + wave) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ swz4(row);
    if (i < 4)
      src[i] = A + (int64_t)min(m0 + row, M - 1) * rowbytes + chunk * 16;
    else
      src[i] = B + (int64_t)min(n0 + row - 256, N - 1) * rowbytes + chunk * 16;
  }
  // Scale DMA: scale tile t = wave*4 + lane/16 (A row tiles 0..7, then B row
  // tiles), bytes (lane%16)*16 of the tile's 256 for the stage's chunk.
  const uint8_t* ssrc;
  {
    const int t = wave * 4 + (lane >> 4);
    const int64_t rt = t < 8 ? min((m0 >> 5) + t, (M - 1) >> 5) : min((n0 >> 5) + t - 8, (N - 1) >> 5);
    ssrc = (t < 8 ? As : Bs) + rt * kchunks * 256 + (lane & 15) * 16;
  }
  auto dma = [&](int kt) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);  // past the end: reload the last stage
    uint8_t* slot = dyn_lds + (kt % kDmaStages) * kDmaStageBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(src[i] + ks * 64, (lds_ptr)(slot + (i * 4 + wave) * 1024),
                                       16, 0, 0);
    __builtin_amdgcn_global_load_lds(ssrc + (ks >> 1) * 256, (lds_ptr)(slot + kDmaCodeBytes + wave * 1024),
                                     16, 0, 0);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](const uint8_t* slot, int sel0) __attribute__((always_inline)) {
    uint32_t sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(slot + kDmaCodeBytes + (wm * 4 + i) * 256 + lane * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(slot + kDmaCodeBytes + (8 + wn * 4 + j) * 256 + lane * 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8 af[TM], bf[TN];
      const int q = s * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        const u32x4 t = *reinterpret_cast<const u32x4*>(slot + row * 64 + ((q ^ swz4(row)) * 16));
        af[i] = i32x8{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = BM + wn * WN + j * 32 + (lane & 31);
        const u32x4 t = *reinterpret_cast<const u32x4*>(slot + row * 64 + ((q ^ swz4(row)) * 16));
        bf[j] = i32x8{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
      }
      const int sh = 8 * (sel0 + s);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[i], bf[j], acc[i][j], 4, 4, 0, (int)(sa[i] >> sh), 0, (int)(sb[j] >> sh));
    }
  };

  if (kt0 < kt1) {
    dma(kt0);
    dma(kt0 + 1);
    dma(kt0 + 2);
    for (int kt = kt0; kt < kt1; ++kt) {
      // wait for this wave's DMA of stage kt: 18 later loads may stay in
      // flight (gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt and
      // lgkmcnt at their maxima), and for its own LDS reads of stage kt-1
      __builtin_amdgcn_s_waitcnt((18 & 15) | (7 << 4) | (0 << 8) | ((18 >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      dma(kt + 3);
      compute(dyn_lds + (kt % kDmaStages) * kDmaStageBytes, (kt & 1) * 2);
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));  // vmcnt(0)
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (row < M && col < N) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e]);
        }
      }
}

// The DMA kernel uses more than the default 64 KB of LDS; raise its limit once.
template <int YDT, bool PARTIAL>
hipError_t dma_lds_attr(size_t bytes) {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_mx_dma_kernel<YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return status;
}

// Y = sum over splits of the fp32 partials (fixed order), times gscale.
template <int YDT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 int splits, int M, int N,
                                                                 void* __restrict__ Y,
                                                                 int64_t ldy) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * total + i];
    const int row = (int)(i / N), col = (int)(i - (int64_t)row * N);
    store_out<YDT>(Y, ldy, row, col, s);
  }
}

// ------------------------------------------------------------------ NVFP4
// Block tile 128 x 128, K-stage of 64 (4 NVFP4 blocks), four waves of 64 x 64
// built from 16x16x32 fp16 MFMA tiles.  Each thread dequantizes one 16-byte
// chunk (32 elements, two blocks) of A and one of B per stage into LDS.
template <int YDT>
__global__ __launch_bounds__(kThreads) void gemm_nv_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ ags,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ bgs,
    void* __restrict__ Y, int64_t ldy, int M, int N, int K, int tiles_n) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, TM = WM / 16, TN = WN / 16;
  constexpr int ROWB = 128;  // bytes per LDS row: 64 fp16
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - (blockIdx.x / tiles_n) * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int64_t srow = K / 16;
  const int KT = K / 64;

  // this thread's chunk: row c >> 1, half c & 1 (32 elements = blocks 2h, 2h+1)
  const int c_row = tid >> 1, c_half = tid & 1;
  const int a_row = min(m0 + c_row, M - 1), b_row = min(n0 + c_row, N - 1);
  u32x4 ra, rb;
  uint32_t sca, scb;
  auto gload = [&](int kt) __attribute__((always_inline)) {
    ra = *reinterpret_cast<const u32x4*>(A + (int64_t)a_row * rowbytes + kt * 32 + c_half * 16);
    rb = *reinterpret_cast<const u32x4*>(B + (int64_t)b_row * rowbytes + kt * 32 + c_half * 16);
    sca = *reinterpret_cast<const uint16_t*>(As + (int64_t)a_row * srow + kt * 4 + c_half * 2);
    scb = *reinterpret_cast<const uint16_t*>(Bs + (int64_t)b_row * srow + kt * 4 + c_half * 2);
  };
  // 16 bytes of codes + two E4M3 scale bytes -> 32 fp16 values -> 4 LDS chunks.
  auto expand = [&](u32x4 codes, uint32_t sc2, uint8_t* dst_row) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const _Float16 s = (_Float16)e4m3_value((sc2 >> (8 * blk)) & 0xFFu);
      const f16x2 s2 = {s, s};
#pragma unroll
      for (int dwi = 0; dwi < 2; ++dwi) {
        const uint32_t w = codes[blk * 2 + dwi];
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w >> (8 * j), 1.0f, 0);
          v = v * s2;
          o[j] = __builtin_bit_cast(uint32_t, v);
        }
        const int chunk = c_half * 4 + blk * 2 + dwi;  // 8 fp16 per chunk
        const int row = c_row;
        *reinterpret_cast<u32x4*>(dst_row + ((chunk ^ swz8(row)) * 16)) = o;
      }
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    expand(ra, sca, &lds[buf][c_row * ROWB]);
    expand(rb, scb, &lds[buf][BM * ROWB + c_row * ROWB]);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (KT > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f16x8 af[TM], bf[TN];
      const int chunk = s * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int row = wm * WM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const f16x8*>(&lds[buf][row * ROWB + ((chunk ^ swz8(row)) * 16)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int row = wn * WN + j * 16 + (lane & 15);
        bf[j] = *reinterpret_cast<const f16x8*>(&lds[buf][BM * ROWB + row * ROWB + ((chunk ^ swz8(row)) * 16)]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  const float g = (*ags) * (*bgs);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + e;
        const int col = n0 + wn * WN + j * 16 + (lane & 15);
        if (row < M && col < N) store_out<YDT>(Y, ldy, row, col, acc[i][j][e] * g);
      }
}

struct MxPlan {
  int cfg;     // 0: 256x256, 1: 128x128, 2: 32x128
  int splits;  // split-K factor (1 = none)
  int kt_per;  // K-stages per split
};

MxPlan plan_mx(int64_t M, int64_t N, int64_t K) {
  MxPlan p{1, 1, (int)(K / 128)};
  if (M >= 1024 && N >= 1024) p.cfg = 0;
  else if (M <= 32) p.cfg = 2;
  else p.cfg = 1;
  const int bm = p.cfg == 0 ? 256 : (p.cfg == 1 ? 128 : 32);
  const int bn = p.cfg == 0 ? 256 : 128;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int KT = (int)(K / 128);
  // split K until there are enough workgroups to cover the chip
  // (only for skinny M, where the partial sums are small next to the weights)
  int splits = 1;
  while (M <= 256 && tiles * splits < 512 && splits < 8 && KT / (splits * 2) >= 4) splits *= 2;
  p.splits = splits;
  p.kt_per = (KT + splits - 1) / splits;
  p.kt_per += p.kt_per & 1;  // slices start on a 256-K scale chunk
  return p;
}

}  // namespace

namespace fp4lib {

size_t gemm_mx_workspace(int64_t M, int64_t N, int64_t K) {
  MxPlan p = plan_mx(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const uint8_t* b, const uint8_t* bs, void* y, int ydt, int64_t ldy,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  MxPlan p = plan_mx(M, N, K);
  const int kchunks = (int)mx_gemm_kchunks(K);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_mx_workspace(M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
#define FP4_GMX(BM_, BN_, WM_, WN_)                                                                 \
  do {                                                                                              \
    const int tiles_n = (int)((N + BN_ - 1) / BN_);                                                 \
    dim3 grid((unsigned)(((M + BM_ - 1) / BM_) * tiles_n), (unsigned)splits);                      \
    const int nt = 64 * (BM_ / WM_) * (BN_ / WN_);                                                  \
    if (split)                                                                                      \
      gemm_mx_kernel<BM_, BN_, WM_, WN_, FP4_DT_F32, true><<<grid, nt, 0, st>>>(                    \
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);           \
    else if (ydt == FP4_DT_F32)                                                                     \
      gemm_mx_kernel<BM_, BN_, WM_, WN_, FP4_DT_F32, false><<<grid, nt, 0, st>>>(                   \
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);           \
    else                                                                                            \
      gemm_mx_kernel<BM_, BN_, WM_, WN_, FP4_DT_BF16, false><<<grid, nt, 0, st>>>(                  \
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);           \
  } while (0)
  if (p.cfg == 0) {
    const int tiles_n = (int)((N + 255) / 256);
    dim3 grid((unsigned)(((M + 255) / 256) * tiles_n), (unsigned)splits);
    const size_t lds = (size_t)kDmaStages * kDmaStageBytes;
    hipError_t e;
    if (split) {
      if ((e = dma_lds_attr<FP4_DT_F32, true>(lds)) != hipSuccess) return e;
      gemm_mx_dma_kernel<FP4_DT_F32, true><<<grid, 256, lds, st>>>(
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
    } else if (ydt == FP4_DT_F32) {
      if ((e = dma_lds_attr<FP4_DT_F32, false>(lds)) != hipSuccess) return e;
      gemm_mx_dma_kernel<FP4_DT_F32, false><<<grid, 256, lds, st>>>(
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
    } else {
      if ((e = dma_lds_attr<FP4_DT_BF16, false>(lds)) != hipSuccess) return e;
      gemm_mx_dma_kernel<FP4_DT_BF16, false><<<grid, 256, lds, st>>>(
          a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
    }
  } else if (p.cfg == 1) {
    FP4_GMX(128, 128, 64, 64);
  } else {
    FP4_GMX(32, 128, 32, 32);
  }
#undef FP4_GMX
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  int64_t total = M * N;
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 8192) g = 8192;
  if (ydt == FP4_DT_F32)
    splitk_reduce_kernel<FP4_DT_F32><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy);
  else
    splitk_reduce_kernel<FP4_DT_BF16><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy);
  return hipGetLastError();
}

size_t gemm_nv_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_nv(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                          void* y, int ydt, int64_t ldy, void*, size_t, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const int tiles_n = (int)((N + 127) / 128);
  const unsigned grid = (unsigned)(((M + 127) / 128) * tiles_n);
  if (ydt == FP4_DT_F32)
    gemm_nv_kernel<FP4_DT_F32><<<grid, kThreads, 0, st>>>(a, as, ags, b, bs, bgs, y, ldy, (int)M,
                                                          (int)N, (int)K, tiles_n);
  else
    gemm_nv_kernel<FP4_DT_BF16><<<grid, kThreads, 0, st>>>(a, as, ags, b, bs, bgs, y, ldy, (int)M,
                                                           (int)N, (int)K, tiles_n);
  return hipGetLastError();
}

}  // namespace fp4lib
