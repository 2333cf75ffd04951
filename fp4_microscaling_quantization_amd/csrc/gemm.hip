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
// (selected with the instruction's byte select).  Large tiles (256 x 256)
// stream K-stages of 256 through two LDS slots (gemm_mx2_kernel); the other
// plans use K-stages of 128 and a deeper ring (gemm_mx_kernel).
//
// NVFP4 has no E4M3-scaled MFMA: each K-tile is dequantized into LDS as fp16,
// e2m1 * e4m3 being exact in fp16 (at most 6 significant bits, magnitudes in
// [2^-10, 2688]), and multiplied on the fp16 MFMA; the fp32 tensor scales
// multiply the accumulator in the epilogue ("Portable FP4 Quantization for
// Heterogeneous Accelerators", section 2.5: conversion fused with GEMM entry
// instead of materialising a full-precision copy).
#include <type_traits>

#include "fp4_device.h"
#include "launch.h"

using namespace fp4k;

namespace {

constexpr int kThreads = 256;
// Most K-slices a split-K plan uses.
constexpr int kMaxSplits = 16;

// XOR swizzle of 16-byte chunks within a 64-byte LDS row (4 chunks): four
// consecutive rows share a 256-byte bank line, so rows 4i .. 4i+3 keep their
// chunk order and each group of four rows rotates it by i.  The fragment reads
// (lane l: row l % 32, one chunk) then see no bank conflicts (measured with
// SQ_LDS_BANK_CONFLICT on gfx950; a rotation by bits 1-2 of the row was 2-way).
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
// Same for 128-byte rows (8 chunks).
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
// Orders a wave's LDS writes before its own later LDS reads of other lanes'
// data (no other wave touches the region).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// 128-byte rows read as 32x32x64 MFMA fragments (lane l: row l % 32): a
// rotation of the eight 16-byte chunks that depends on row % 32 only, so all
// fragments of a lane share one chunk offset; conflict-free for 16 (and 8)
// consecutive rows reading the same chunk.
__device__ __forceinline__ int swz32(int row) { return (row ^ ((row >> 3) & 3)) & 7; }

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

// MXFP4 GEMM.  Block tile BM x BN, four or eight waves each owning a WM x WN
// sub-tile of 32x32 MFMA tiles (v_mfma_scale_f32_32x32x64_f8f6f4, accumulators in
// AGPRs), K-stages of 128 (64 bytes of codes per row, two MFMA steps).
//
// Codes and scale tiles stream straight from global memory into an NS-slot
// LDS ring with global_load_lds_dwordx4 (no staging registers).  A slot holds
// [A codes BM x 64 B | B codes BN x 64 B | A scale tiles | B scale tiles]
// (one 256-byte GEMM-layout scale tile per 32 rows for the stage's 256-K
// chunk), rounded up to whole rounds of 1 KB per wave: in each round every thread moves
// 16 bytes, and the source of each (thread, round) is fixed at kernel start;
// code rows are 64-byte LDS rows whose 16-byte chunks are XOR-swizzled by
// choosing the source chunk.  Every iteration issues the same number of DMAs
// (stages past the end re-load the last stage into the slot that is free), so
// one exact wait (the later stages' DMAs may stay in flight) and one barrier
// per stage suffice.  Fragment reads for the next MFMA step and the DMAs are
// slotted between the MFMAs.  With PARTIAL, blockIdx.y selects a K-slice of
// an even number of stages and fp32 partial sums go to the workspace.
template <int BM, int BN, int WM, int WN, int NS>
struct MxCfg {
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int B_CODES = BM * 64;
  static constexpr int A_SC = B_CODES + BN * 64;
  static constexpr int B_SC = A_SC + (BM / 32) * 256;
  static constexpr int USED = B_SC + (BN / 32) * 256;
  static constexpr int NW = (BM / WM) * (BN / WN);          // waves per workgroup
  static constexpr int RB = NW * 1024;                      // bytes per DMA round
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  static constexpr int LDS = NS * STAGE;
  // Waves whose share of the last round is all slot padding skip that DMA
  // (and count one DMA less per stage in their waits).
  static constexpr int LAST_W = (USED - (ROUNDS - 1) * RB + 1023) / 1024;
  static constexpr bool SKIP = LAST_W < NW;
  // The last round holds only the scale tiles (and padding).  A scale tile
  // covers 256 K, two stages, so odd stages skip that round and keep the
  // even stage's scale registers; with NS - 2 even, every wait then counts
  // the same number of DMAs.
  static constexpr bool SC_ROUND = (BM + BN) * 64 == (ROUNDS - 1) * RB && (NS - 2) % 2 == 0;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NS >= 3 && (NS - 1) * ROUNDS <= 63, "vmcnt range");
};

// Operand registers of one 64-K MFMA step of a wave: TM A and TN B fragments
// (16 bytes each) and their scale dwords.
template <int TM, int TN>
struct MxFrags {
  u32x4 a[TM], b[TN];
};
template <int TM, int TN>
struct MxScales {
  uint32_t a[TM], b[TN];
};

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (lds must be the same for the whole wave).  Kept out of the kernel templates:
// the builtin must not see template-dependent arguments.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
}

// The scaled MFMA (E2M1 x E2M1, fp32 accumulate) with byte 0 of each scale
// dword as the E8M0 scale.  A non-template wrapper: the builtin must not see
// template-dependent arguments.
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// The same with the instruction's byte select choosing byte SEL of each scale
// dword (one wrapper per byte: the builtin takes constants only).
__device__ __forceinline__ f32x16 mfma_mx_b0(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x16 mfma_mx_b1(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 1, sa, 1, sb);
}
__device__ __forceinline__ f32x16 mfma_mx_b2(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 2, sa, 2, sb);
}
__device__ __forceinline__ f32x16 mfma_mx_b3(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 3, sa, 3, sb);
}

// gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; a field at its maximum does not wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

template <int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL>
__global__ __launch_bounds__((MxCfg<BM, BN, WM, WN, NS>::NW * 64)) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, void* __restrict__ Y, int64_t ldy, int M, int N, int K,
    int kchunks, int tiles_n, int kt_per_split, float* __restrict__ part, int bt) {
  using C = MxCfg<BM, BN, WM, WN, NS>;
  constexpr int TM = C::TM, TN = C::TN, ROUNDS = C::ROUNDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / (BN / WN), wn = wave % (BN / WN);
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // DMA sources of this thread, one per round: slot byte p = r*RB + tid*16,
  // and the bytes a stage advances them (0: a scale round, which advances one
  // 256-byte tile every two stages).  Tiled B codes (bt): a stage is the next
  // 8 KB tile of the row panel.
  const uint8_t* src[ROUNDS];
  uint32_t cadv[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < C::B_CODES) {
      const int row = p >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = A + (int64_t)min(m0 + row, M - 1) * rowbytes + chunk * 16;
      cadv[r] = 64;
    } else if (p < C::A_SC) {
      const int row = (p - C::B_CODES) >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + code_offset(min(n0 + row, N - 1), chunk * 16, rowbytes, bt != 0);
      cadv[r] = bt ? 8192 : 64;
    } else if (p < C::B_SC) {
      const int t = (p - C::A_SC) >> 8;
      src[r] = As + (int64_t)min((m0 >> 5) + t, (M - 1) >> 5) * kchunks * 256 + (p & 255);
      cadv[r] = 0;
    } else if (p < C::USED) {
      const int t = (p - C::B_SC) >> 8;
      src[r] = Bs + (int64_t)min((n0 >> 5) + t, (N - 1) >> 5) * kchunks * 256 + (p & 255);
      cadv[r] = 0;
    } else {  // slot padding: any valid address
      src[r] = As + (p & 255);
      cadv[r] = 0;
    }
  }
  auto slot_of = [&](int kt) __attribute__((always_inline)) {
    return dyn_lds + (kt % NS) * C::STAGE;
  };
  // A stage's DMA goes out in two parts: rounds [0, H) in the second half of
  // one iteration and rounds [H, ROUNDS) in the first half of the next, so
  // that each half iteration asks the address unit for about half a stage.
  constexpr int H = ROUNDS / 2;
  auto dma_head = [&](int kt) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);  // past the end: reload the last stage
    uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int r = 0; r < H; ++r)
      dma16(src[r] + (cadv[r] ? (int64_t)ks * cadv[r] : (int64_t)(ks >> 1) * 256), slot + r * C::RB + wave * 1024);
  };
  // SHORT: this wave's part of the last round is slot padding, not loaded;
  // skip_last: an odd stage's scale round (SC_ROUND), not loaded either.
  auto dma_tail = [&](int kt, auto short_tag, bool skip_last) __attribute__((always_inline)) {
    constexpr int RE = decltype(short_tag)::value ? ROUNDS - 1 : ROUNDS;
    const int ks = min(kt, kt1 - 1);
    uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int r = H; r < RE; ++r) {
      if (r == ROUNDS - 1 && skip_last) continue;
      dma16(src[r] + (cadv[r] ? (int64_t)ks * cadv[r] : (int64_t)(ks >> 1) * 256), slot + r * C::RB + wave * 1024);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  using Frags = MxFrags<TM, TN>;
  using Scales = MxScales<TM, TN>;
  auto read_frags = [&](const uint8_t* slot, int s, Frags& f) __attribute__((always_inline)) {
    const int q = s * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 32 + (lane & 31);
      f.a[i] = *reinterpret_cast<const u32x4*>(slot + row * 64 + ((q ^ swz4(row)) * 16));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + j * 32 + (lane & 31);
      f.b[j] = *reinterpret_cast<const u32x4*>(slot + C::B_CODES + row * 64 + ((q ^ swz4(row)) * 16));
    }
  };
  auto read_scales = [&](const uint8_t* slot, Scales& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sc.a[i] = *reinterpret_cast<const uint32_t*>(slot + C::A_SC + ((wm * WM) / 32 + i) * 256 + lane * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sc.b[j] = *reinterpret_cast<const uint32_t*>(slot + C::B_SC + ((wn * WN) / 32 + j) * 256 + lane * 4);
  };
  auto mfmas = [&](const Frags& f, const Scales& sc, int sel) __attribute__((always_inline)) {
    const int sh = 8 * sel;  // byte of the scale dword for this 64-K step
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x8 av = {(int)f.a[i][0], (int)f.a[i][1], (int)f.a[i][2], (int)f.a[i][3], 0, 0, 0, 0};
        const i32x8 bv = {(int)f.b[j][0], (int)f.b[j][1], (int)f.b[j][2], (int)f.b[j][3], 0, 0, 0, 0};
        acc[i][j] = mfma_mx(av, bv, acc[i][j], (int)(sc.a[i] >> sh), (int)(sc.b[j] >> sh));
      }
  };

  constexpr int NMF = TM * TN;             // MFMAs per 64-K step
  constexpr int NRD = TM + TN;             // fragment reads per step
  constexpr int NSC = (TM + TN + 1) / 2;   // scale reads (paired dwords)
  constexpr int NVA = ROUNDS - H;          // DMAs in the first half iteration
  constexpr int NVB = H;                   // DMAs in the second half

  // The ring, for waves that load every round of a stage or all but the last
  // (SHORT).  PAIR: DMAs of two consecutive stages.
  auto ring = [&](auto short_tag) __attribute__((always_inline)) {
    constexpr bool SHORT = decltype(short_tag)::value;
    constexpr bool SR = C::SC_ROUND;
    constexpr int PAIR = SHORT ? 2 * (ROUNDS - 1) : (SR ? 2 * ROUNDS - 1 : 2 * ROUNDS);
    constexpr int AFTER = (NS - 2) / 2 * PAIR + ((NS - 2) % 2) * (SHORT ? ROUNDS - 1 : ROUNDS);
    // In iteration kt the registers hold step 0 of stage kt (F0, S).  First
    // half: step 1's reads and the tail of stage kt+NS-1's DMA go out with
    // step 0's MFMAs.  Each wave then waits for its own DMA of stage kt+1 and
    // its LDS reads, and the workgroup syncs (stage kt+1 complete everywhere,
    // slot kt read by nobody).  Second half: the head of stage kt+NS's DMA
    // into slot kt and stage kt+1's step-0 (and, for an even stage, scale)
    // reads go out with step 1's MFMAs.  Slices start at even stages.
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
      dma_head(kt0 + i);
      dma_tail(kt0 + i, short_tag, SR && (i & 1));
    }
    dma_head(kt0 + NS - 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(AFTER + H, 15));
    __builtin_amdgcn_s_barrier();
    Frags F0, F1;
    Scales S, S1;
    read_frags(slot_of(kt0), 0, F0);
    read_scales(slot_of(kt0), S);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    // ODD: parity of kt (used only with SR)
    auto iter = [&](int kt, auto odd_tag) __attribute__((always_inline)) {
      constexpr bool ODD = decltype(odd_tag)::value;
      constexpr bool TAIL_SKIP = SR && (((ODD ? 1 : 0) + NS - 1) & 1);
      constexpr bool READ_SC = !SR || ODD;  // stage kt+1 even: its scale tiles
      const int sel0 = (kt & 1) * 2;
      read_frags(slot_of(kt), 1, F1);
      dma_tail(kt + NS - 1, short_tag, TAIL_SKIP);
      mfmas(F0, S, sel0);
#pragma unroll
      for (int k = 0; k < NMF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
        if (k < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
        if (k < NVA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // DMA
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(AFTER, 0));  // DMAs after stage kt+1
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      dma_head(kt + NS);
      read_frags(slot_of(kt + 1), 0, F0);
      if constexpr (READ_SC) read_scales(slot_of(kt + 1), S1);
      mfmas(F1, S, sel0 + 1);
#pragma unroll
      for (int k = 0; k < NMF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
        if (k < NRD + (READ_SC ? NSC : 0)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (k < NVB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (READ_SC) {
#pragma unroll
        for (int i = 0; i < TM; ++i) S.a[i] = S1.a[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) S.b[j] = S1.b[j];
      }
    };
    if constexpr (SR) {
      int kt = kt0;
      for (; kt + 1 < kt1; kt += 2) {
        iter(kt, std::false_type{});
        iter(kt + 1, std::true_type{});
      }
      if (kt < kt1) iter(kt, std::false_type{});  // K % 256 == 128: a last, even stage
    } else {
      for (int kt = kt0; kt < kt1; ++kt) iter(kt, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  };
  if (kt0 < kt1) {
    if constexpr (C::SKIP) {
      if (__builtin_amdgcn_readfirstlane(wave) >= C::LAST_W)
        ring(std::true_type{});
      else
        ring(std::false_type{});
    } else {
      ring(std::false_type{});
    }
  }

  // Epilogue: whole tiles store without bounds checks.
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (full || (row < M && col < N)) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e]);
        }
        // one accumulator tile at a time (keeps the register footprint small)
        if (e == 15) __builtin_amdgcn_sched_barrier(0);
      }
}

// MXFP4 GEMM with K-stages of 256: each stage holds 128 bytes of codes per
// row (whole 128-byte lines, so every DMA instruction reads 8 rows x 128 B)
// and one 256-byte GEMM-layout scale tile per 32 rows; two LDS slots (the
// stage being multiplied and the one being loaded).  Requires K % 256 == 0.
template <int BM, int BN, int WM, int WN>
struct Mx2Cfg {
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int ROWB = 128;
  static constexpr int B_CODES = BM * ROWB;
  static constexpr int A_SC = B_CODES + BN * ROWB;
  static constexpr int B_SC = A_SC + (BM / 32) * 256;
  static constexpr int USED = B_SC + (BN / 32) * 256;
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int RB = NW * 1024;
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int LAST_W = (USED - (ROUNDS - 1) * RB + 1023) / 1024;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(LDS <= 160 * 1024, "two stages fit the LDS");
  static_assert(A_SC % RB == 0, "code rounds and scale rounds do not share a round");
};

template <int BM, int BN, int WM, int WN, int YDT, bool PARTIAL>
__global__ __launch_bounds__((Mx2Cfg<BM, BN, WM, WN>::NW * 64)) void gemm_mx2_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, void* __restrict__ Y, int64_t ldy, int M, int N, int K,
    int kchunks, int tiles_n, int ks_per_split, float* __restrict__ part, int vec_out, int bt) {
  using C = Mx2Cfg<BM, BN, WM, WN>;
  constexpr int TM = C::TM, TN = C::TN, ROUNDS = C::ROUNDS;
  constexpr int CR = C::A_SC / C::RB;  // rounds of codes (A, then B)
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (BN / WN), wn = wave % (BN / WN);
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t rowbytes = (uint32_t)(K / 2);
  const int KS_total = K / 256;
  const int ks0 = PARTIAL ? blockIdx.y * ks_per_split : 0;
  const int ks1 = PARTIAL ? min(KS_total, ks0 + ks_per_split) : KS_total;

  // DMA sources: 32-bit offsets from A or B for the code rounds (a stage
  // advances them by 128 bytes, or by two 8 KB tiles for tiled B codes), full
  // pointers for the scale rounds (a stage advances them by one 256-byte tile).
  static_assert(C::B_CODES % C::RB == 0, "a code round is all A or all B");
  uint32_t coff[CR];
#pragma unroll
  for (int r = 0; r < CR; ++r) {
    const int p = r * C::RB + tid * 16;
    const bool isa = p < C::B_CODES;
    const int row = (isa ? p : p - C::B_CODES) >> 7, chunk = ((p >> 4) & 7) ^ swz32(row);
    const int64_t grow = min((isa ? m0 : n0) + row, (isa ? M : N) - 1);
    coff[r] = (uint32_t)code_offset(grow, chunk * 16, rowbytes, !isa && bt != 0);
  }
  const uint32_t badv = bt ? 16384u : 128u;
  const uint8_t* ssrc[ROUNDS - CR];
#pragma unroll
  for (int r = CR; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < C::B_SC) {
      const int t = (p - C::A_SC) >> 8;
      ssrc[r - CR] = As + (int64_t)min((m0 >> 5) + t, (M - 1) >> 5) * kchunks * 256 + (p & 255);
    } else if (p < C::USED) {
      const int t = (p - C::B_SC) >> 8;
      ssrc[r - CR] = Bs + (int64_t)min((n0 >> 5) + t, (N - 1) >> 5) * kchunks * 256 + (p & 255);
    } else {
      ssrc[r - CR] = As + (p & 255);
    }
  }
  // rounds [r0, r1) of stage ks into its slot; FULL: this wave loads the last
  // round (otherwise that round is slot padding for it)
  auto dma_stage = [&](int ks, int r0, int r1, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    uint8_t* slot = dyn_lds + (ks & 1) * C::STAGE + wave * 1024;
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      if (!FULL && r == ROUNDS - 1) continue;
      if (r < CR)
        dma16((r * C::RB < C::B_CODES ? A : B) +
                  (coff[r] + (uint32_t)ks * (r * C::RB < C::B_CODES ? 128u : badv)),
              slot + r * C::RB);
      else
        dma16(ssrc[r - CR] + ks * 256, slot + r * C::RB);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  using Frags = MxFrags<TM, TN>;
  using Scales = MxScales<TM, TN>;
  // every fragment row of this lane is = lane (mod 32): one swizzle
  const int lrow = lane & 31, sw = swz32(lrow), half = lane >> 5;
  const int a_base = (wm * WM + lrow) * 128, b_base = C::B_CODES + (wn * WN + lrow) * 128;
  auto read_frags = [&](const uint8_t* slot, int s, Frags& f) __attribute__((always_inline)) {
    const int off = (((2 * s + half) ^ sw) * 16);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      f.a[i] = *reinterpret_cast<const u32x4*>(slot + a_base + off + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      f.b[j] = *reinterpret_cast<const u32x4*>(slot + b_base + off + j * 32 * 128);
  };
  auto read_scales = [&](const uint8_t* slot, Scales& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sc.a[i] = *reinterpret_cast<const uint32_t*>(slot + C::A_SC + ((wm * WM) / 32 + i) * 256 + lane * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sc.b[j] = *reinterpret_cast<const uint32_t*>(slot + C::B_SC + ((wn * WN) / 32 + j) * 256 + lane * 4);
  };
  auto mfmas = [&](const Frags& f, const Scales& sc, int sel) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x8 av = {(int)f.a[i][0], (int)f.a[i][1], (int)f.a[i][2], (int)f.a[i][3], 0, 0, 0, 0};
        const i32x8 bv = {(int)f.b[j][0], (int)f.b[j][1], (int)f.b[j][2], (int)f.b[j][3], 0, 0, 0, 0};
        const int sa = (int)sc.a[i], sb = (int)sc.b[j];
        if (sel == 0) acc[i][j] = mfma_mx_b0(av, bv, acc[i][j], sa, sb);
        else if (sel == 1) acc[i][j] = mfma_mx_b1(av, bv, acc[i][j], sa, sb);
        else if (sel == 2) acc[i][j] = mfma_mx_b2(av, bv, acc[i][j], sa, sb);
        else acc[i][j] = mfma_mx_b3(av, bv, acc[i][j], sa, sb);
      }
  };
  constexpr int NMF = TM * TN;
  constexpr int NRD = TM + TN;
  // The stage barrier sits after step 2: by then every wave holds step 3's
  // fragments in registers, so the stage's slot is free, and (each wave
  // having waited for its own DMAs) the next stage has landed.  Step 3's MFMAs
  // then cover the next stage's first fragment reads, its scale reads (issued
  // after them) and the first E3 rounds of the stage after next, into the
  // freed slot; that stage's remaining rounds go out in two parts with steps
  // 0 and 1 of the next stage.  The barrier after the next stage's step 2
  // waits for all of them: four, three and two steps after their issue.
  // Measured against a barrier after step 3 (and three DMA parts within the
  // stage): 4-8 % less time on every 256x256 shape.
  constexpr int E3 = 4;
  constexpr int H = (E3 + ROUNDS + 1) / 2;
  static_assert(E3 < ROUNDS, "step 3's rounds are full rounds for every wave");

  auto ring = [&](auto full_tag) __attribute__((always_inline)) {
    dma_stage(ks0, 0, ROUNDS, full_tag);
    if (ks0 + 1 < ks1) {
      dma_stage(ks0 + 1, 0, E3, full_tag);
      // stage ks0 landed for this wave: only ks0 + 1's first E3 rounds in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(E3, 15));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    }
    __builtin_amdgcn_s_barrier();
    Frags F0, F1;
    Scales S;
    read_frags(dyn_lds, 0, F0);
    read_scales(dyn_lds, S);
    for (int ks = ks0; ks < ks1; ++ks) {
      const uint8_t* slot = dyn_lds + (ks & 1) * C::STAGE;
      const uint8_t* nslot = dyn_lds + ((ks + 1) & 1) * C::STAGE;
      const bool next = ks + 1 < ks1;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frags& cur = (s & 1) ? F1 : F0;
        Frags& nxt = (s & 1) ? F0 : F1;
        if (s < 3) read_frags(slot, s + 1, nxt);
        if (s == 3) {
          // past the last stage these reads fetch a stale slot (unused) and
          // the DMA re-loads the last stage (its data, or a slot nobody reads
          // again); unconditional, which keeps the register allocation spill-free
          read_frags(nslot, 0, F0);
          dma_stage(min(ks + 2, ks1 - 1), 0, E3, full_tag);
        }
        if (s == 0 && next) dma_stage(ks + 1, E3, H, full_tag);
        if (s == 1 && next) dma_stage(ks + 1, H, ROUNDS, full_tag);
        mfmas(cur, S, s);
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (s < 3 && k < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (s < 2 && k < 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (s == 2) {
          // stage ks + 1 complete (this wave's DMAs, then everyone's) and
          // slot ks read by nobody any more
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // after step 3's MFMAs have taken the current scales
      read_scales(nslot, S);
    }
    // the last stages' re-load DMAs land before the ring is reused
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  };
  if (ks0 < ks1) {
    if (wave < C::LAST_W)
      ring(std::true_type{});
    else
      ring(std::false_type{});
  }

  const bool full = m0 + BM <= M && n0 + BN <= N;
  if constexpr (!PARTIAL && YDT == FP4_DT_BF16) {
    if (full && vec_out) {
      // bf16 tile through LDS (the ring is free once every wave is past its
      // last stage): each wave writes its WM x WN tile row-major with a
      // 16-byte row pad, then stores whole 16-byte row pieces (8 rows x 128 B
      // per instruction) instead of 2-byte scattered stores.
      constexpr int PITCH = WN * 2 + 16;
      static_assert(C::NW * WM * PITCH <= C::LDS, "staging fits the ring");
      __builtin_amdgcn_s_barrier();
      uint8_t* st = dyn_lds + wave * (WM * PITCH);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            const int col = j * 32 + (lane & 31);
            *reinterpret_cast<uint16_t*>(st + row * PITCH + col * 2) =
                (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
          }
      wave_lds_fence();
      constexpr int CPR = WN * 2 / 16;  // 16-byte pieces per row
      uint16_t* yb = static_cast<uint16_t*>(Y);
#pragma unroll
      for (int p = 0; p < WM * CPR / 64; ++p) {
        const int r = p * (64 / CPR) + lane / CPR, c = lane % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * PITCH + c * 16);
        *reinterpret_cast<u32x4*>(yb + (int64_t)(m0 + wm * WM + r) * ldy + n0 + wn * WN + c * 8) = v;
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (full || (row < M && col < N)) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e]);
        }
        if (e == 15) __builtin_amdgcn_sched_barrier(0);
      }
}

// ------------------------------------------------------------------ NVFP4
// NVFP4 GEMM on the fp16 MFMA (v_mfma_f32_32x32x16_f16), same ring as the
// MXFP4 kernel: FP4 codes and E4M3 scales stream into LDS by DMA and each
// wave expands its own fragments to fp16 in registers (e2m1 * e4m3 is exact
// in fp16: at most 6 significant bits, magnitudes in [2^-10, 2688]), so LDS
// holds 4-bit codes and the expansion overlaps the MFMAs.  A stage is K = 128
// (64 bytes of codes per row); the per-row scale chunk is 16 bytes (16 blocks,
// K = 256), reloaded with each stage of the pair.  Requires K % 256 == 0.
//
// K order inside an MFMA is free as long as A and B agree: a lane reads the
// same 16 bytes (32 codes, K = 32h .. 32h + 31 of the 64-K step, h = lane /
// 32) as in the MXFP4 kernel and feeds dword t of them to MFMA t of the step,
// for A rows and B columns alike.  The fp32 tensor scales multiply the
// accumulators in the epilogue.
template <int BM, int BN, int WM, int WN, int NS, int FMT = FP4_FMT_NVFP4, int KG = 1>
struct NvCfg {
  // MX: E8M0 scales in the GEMM layout (one 256-byte tile per 32 rows per
  // 256 K, re-loaded with each stage of the pair); NV: each row's 16 E4M3
  // scales of the 256-K chunk.
  static constexpr bool MX = fmt_mx(FMT);
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int B_CODES = BM * 64;
  static constexpr int A_SC = B_CODES + BN * 64;
  static constexpr int B_SC = A_SC + (MX ? BM * 8 : BM * 16);
  static constexpr int USED = B_SC + (MX ? BN * 8 : BN * 16);
  static constexpr int SC_ADV = MX ? 256 : 16;  // scale bytes per 256-K chunk and source
  // KG = 2: two groups of waves, each taking one 64-K step of every stage
  // (two waves per SIMD for the small decode tiles), summed at the end
  static constexpr int WPG = (BM / WM) * (BN / WN);  // waves per group
  static constexpr int NW = KG * WPG;
  static constexpr int RB = NW * 1024;
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  // With two groups the A tile of each stage is expanded once per workgroup
  // (one 8-code piece per thread) into one of two 16-bit LDS buffers, two
  // stages ahead of its use, instead of by every wave that reads it.
  static constexpr bool AEXP = KG == 2 && WM == BM;  // every wave reads all BM rows
  static constexpr int ABUF = AEXP ? BM * 256 : 0;  // BM rows x 128 K x 2 bytes
  static constexpr int APIECES = AEXP ? BM * 16 / (NW * 64) : 0;  // 8-code pieces per thread
  static constexpr int LDS = NS * STAGE + 2 * ABUF;
  static constexpr int IN_FLIGHT = (NS - (AEXP ? 3 : 2)) * ROUNDS;
  static_assert(!AEXP || (NS >= 4 && APIECES * NW * 64 == BM * 16), "A expansion: lookahead, whole pieces");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(KG == 1 || KG == 2, "one or two K-step groups");
  static_assert(NS >= 3 && (NS - 1) * ROUNDS <= 63, "vmcnt range");
  static_assert(KG == 1 || WPG * TM * TN * 4096 <= LDS, "the group sum fits the ring");
};

// Two E4M3 codes (bits 0-7 and 8-15 of w) as fp16 / fp32 by the hardware FP8
// conversion: every finite E4M3 value, subnormals included, is exactly an
// fp16 and an fp32 value (checked against the bit construction for all 127
// finite codes), and one instruction replaces a subnormal test per code.
__device__ __forceinline__ f16x2 e4m3x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }

__device__ __forceinline__ f32x16 mfma_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight E2M1 codes (one dword, low nibble first) times an fp16 scale.
__device__ __forceinline__ f16x8 expand8(uint32_t w, _Float16 s) {
  const f16x2 s2 = {s, s};
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Eight INT4 codes (two's complement, low nibble first) times an fp16 scale,
// exactly: with u = n + 8 in 0 .. 15, the fp16 word 0x6400 | u is 1024 + u, so
// (word - 1032) is n and n * s (at most 7 significant bits) is exact.  The
// lanes come out in the order 0, 4, 1, 5, 2, 6, 3, 7: a permutation within the
// K range of one MFMA, applied alike to both operands.
__device__ __forceinline__ f16x8 expand8_i4_f16(uint32_t w, _Float16 s) {
  const uint32_t t = w ^ 0x88888888u;
  const f16x2 s2 = {s, s};
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 v0 = (__builtin_bit_cast(f16x2, (t & 0x000F000Fu) | 0x64006400u) - off) * s2;
  const f16x2 v1 = (__builtin_bit_cast(f16x2, ((t >> 4) & 0x000F000Fu) | 0x64006400u) - off) * s2;
  const f16x2 v2 = (__builtin_bit_cast(f16x2, ((t >> 8) & 0x000F000Fu) | 0x64006400u) - off) * s2;
  const f16x2 v3 = (__builtin_bit_cast(f16x2, ((t >> 12) & 0x000F000Fu) | 0x64006400u) - off) * s2;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Eight INT4 codes times an fp32 scale p as bf16, in element order.  Exact
// when n * p has at most 8 significant bits and lies in bf16's range (p a
// power of two or an E4M3 value): the fp32 product's low 16 bits are zero.
__device__ __forceinline__ u32x4 expand8_i4_bf16(uint32_t w, float p) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = int4_value(w, 2 * k) * p, b = int4_value(w, 2 * k + 1) * p;
    r[k] = (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
  }
  return r;
}

template <int TM, int TN>
struct NvFrags {
  u32x4 a[TM], b[TN];
  uint32_t sa[TM], sb[TN];  // two E4M3 scale bytes per fragment (blocks of the lane's 32 codes)
  u32x4 a16[TM][4];         // A already expanded (one 16-bit chunk per MFMA of the step)
};

template <int FMT, int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL, int KG>
__global__ __launch_bounds__((NvCfg<BM, BN, WM, WN, NS, FMT, KG>::NW * 64)) void gemm_nv_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ ags,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ bgs,
    void* __restrict__ Y, int64_t ldy, int M, int N, int K, int tiles_n, int kt_per_split,
    float* __restrict__ part, int bt) {
  using C = NvCfg<BM, BN, WM, WN, NS, FMT, KG>;
  constexpr int TM = C::TM, TN = C::TN, ROUNDS = C::ROUNDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave / C::WPG, wg = wave % C::WPG;  // K-step group, wave in the group
  const int wm = wg / (BN / WN), wn = wg % (BN / WN);
  const int64_t kchunks = K / 256;
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2, srow = K / 16;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // DMA sources and per-stage advances as in gemm_mx_kernel (cadv 0: scales).
  const uint8_t* src[ROUNDS];
  uint32_t cadv[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < C::B_CODES) {
      const int row = p >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = A + (int64_t)min(m0 + row, M - 1) * rowbytes + chunk * 16;
      cadv[r] = 64;
    } else if (p < C::A_SC) {
      const int row = (p - C::B_CODES) >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + code_offset(min(n0 + row, N - 1), chunk * 16, rowbytes, bt != 0);
      cadv[r] = bt ? 8192 : 64;
    } else if (p < C::B_SC) {
      const int q = p - C::A_SC;
      if constexpr (C::MX)
        src[r] = As + (int64_t)min((m0 >> 5) + (q >> 8), (M - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = As + (int64_t)min(m0 + (q >> 4), M - 1) * srow;
      cadv[r] = 0;
    } else if (p < C::USED) {
      const int q = p - C::B_SC;
      if constexpr (C::MX)
        src[r] = Bs + (int64_t)min((n0 >> 5) + (q >> 8), (N - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = Bs + (int64_t)min(n0 + (q >> 4), N - 1) * srow;
      cadv[r] = 0;
    } else {
      src[r] = As;
      cadv[r] = 0;
    }
  }
  auto slot_of = [&](int kt) __attribute__((always_inline)) {
    return dyn_lds + (kt % NS) * C::STAGE;
  };
  constexpr int H = ROUNDS / 2;
  auto dma_head = [&](int kt) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
    uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int r = 0; r < H; ++r)
      dma16(src[r] + (cadv[r] ? (int64_t)ks * cadv[r] : (int64_t)(ks >> 1) * C::SC_ADV), slot + r * C::RB + wave * 1024);
  };
  auto dma_tail = [&](int kt) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
    uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int r = H; r < ROUNDS; ++r)
      dma16(src[r] + (cadv[r] ? (int64_t)ks * cadv[r] : (int64_t)(ks >> 1) * C::SC_ADV), slot + r * C::RB + wave * 1024);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  using Frags = NvFrags<TM, TN>;
  auto abuf_of = [&](int kt) __attribute__((always_inline)) {
    return dyn_lds + NS * C::STAGE + (kt & 1) * C::ABUF;
  };
  // A expansion of stage kt: piece p (thread p, p + 64 NW, ...) is row p / 16,
  // codes 8 (p % 16) .. +7 of the stage, written as 16-bit values to chunk
  // p % 16 of the row rotated by row % 16 (the fragment reads below:
  // conflict-free)
  auto expand_a = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int pc = 0; pc < C::APIECES; ++pc) {
      const uint8_t* slot = slot_of(kt);
      const int p = pc * C::NW * 64 + tid;
      const int row = p >> 4, g = p & 15;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          slot + row * 64 + (((g >> 2) ^ swz4(row)) * 16) + (g & 3) * 4);
      u32x4 v;
      if constexpr (C::MX) {
        const int s = g >> 3, hh = (g >> 2) & 1;
        const uint32_t code = (*reinterpret_cast<const uint32_t*>(slot + C::A_SC + (row >> 5) * 256 +
                                                                  (row & 31) * 4 + hh * 128) >>
                               (8 * (2 * (kt & 1) + s))) & 0xFFu;
        v = expand8_i4_bf16(w, e8m0_value(code));
      } else {
        const _Float16 sc = e4m3x2_f16(slot[C::A_SC + row * 16 + 8 * (kt & 1) + (g >> 1)])[0];
        v = __builtin_bit_cast(u32x4, FMT == FP4_FMT_NVINT4 ? expand8_i4_f16(w, sc) : expand8(w, sc));
      }
      *reinterpret_cast<u32x4*>(abuf_of(kt) + row * 256 + ((g ^ (row & 15)) * 16)) = v;
    }
  };
  // fragments and scale bytes of step s (0, 1) of stage kt
  auto read_step = [&](int kt, int s, Frags& f) __attribute__((always_inline)) {
    const uint8_t* slot = slot_of(kt);
    const int q = s * 2 + (lane >> 5);
    const int sb = 8 * (kt & 1) + 4 * s + 2 * (lane >> 5);  // first block of the lane's 32 codes
    // MX: the lane's scale dword of the tile and the byte of this step
    const int mxo = (lane & 31) * 4 + (lane >> 5) * 128, mxb = 8 * (2 * (kt & 1) + s);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 32 + (lane & 31);
      if constexpr (C::AEXP) {
        const uint8_t* ar = abuf_of(kt) + row * 256;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          f.a16[i][t] = *reinterpret_cast<const u32x4*>(ar + (((8 * s + 4 * (lane >> 5) + t) ^ (lane & 15)) * 16));
        continue;
      }
      f.a[i] = *reinterpret_cast<const u32x4*>(slot + row * 64 + ((q ^ swz4(row)) * 16));
      if constexpr (C::MX)
        f.sa[i] = (*reinterpret_cast<const uint32_t*>(slot + C::A_SC + (row >> 5) * 256 + mxo) >> mxb) & 0xFFu;
      else
        f.sa[i] = *reinterpret_cast<const uint16_t*>(slot + C::A_SC + row * 16 + sb);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + j * 32 + (lane & 31);
      f.b[j] = *reinterpret_cast<const u32x4*>(slot + C::B_CODES + row * 64 + ((q ^ swz4(row)) * 16));
      if constexpr (C::MX)
        f.sb[j] = (*reinterpret_cast<const uint32_t*>(slot + C::B_SC + (row >> 5) * 256 + mxo) >> mxb) & 0xFFu;
      else
        f.sb[j] = *reinterpret_cast<const uint16_t*>(slot + C::B_SC + row * 16 + sb);
    }
  };
  // MFMAs t0 .. t1-1 of a step (one per 16-K piece of the lane's codes)
  auto mfmas = [&](const Frags& f, int t0 = 0, int t1 = 4) __attribute__((always_inline)) {
    if constexpr (C::MX) {
      // MXINT4: q * 2^e exact in bf16, bf16 MFMA
      float pa[TM], pb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) pa[i] = e8m0_value(f.sa[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) pb[j] = e8m0_value(f.sb[j]);
#pragma unroll
      for (int t = t0; t < t1; ++t) {
        u32x4 av[TM], bv[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          av[i] = C::AEXP ? f.a16[i][t] : expand8_i4_bf16(f.a[i][t], pa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = expand8_i4_bf16(f.b[j][t], pb[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16(av[i], bv[j], acc[i][j]);
      }
      return;
    }
    f16x2 sa[TM], sbv[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = e4m3x2_f16(f.sa[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) sbv[j] = e4m3x2_f16(f.sb[j]);
#pragma unroll
    for (int t = t0; t < t1; ++t) {
      f16x8 av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        av[i] = C::AEXP ? __builtin_bit_cast(f16x8, f.a16[i][t])
                : FMT == FP4_FMT_NVINT4 ? expand8_i4_f16(f.a[i][t], sa[i][t >> 1])
                                        : expand8(f.a[i][t], sa[i][t >> 1]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = FMT == FP4_FMT_NVINT4 ? expand8_i4_f16(f.b[j][t], sbv[j][t >> 1]) : expand8(f.b[j][t], sbv[j][t >> 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f16(av[i], bv[j], acc[i][j]);
    }
  };

  if constexpr (KG == 1) {
    if (kt0 < kt1) {
      // Same schedule as the MXFP4 kernel: step 1's reads and the tail of
      // stage kt+NS-1's DMA with step 0's MFMAs; wait for stage kt+1 and
      // sync; the head of stage kt+NS's DMA and stage kt+1's step-0 reads
      // with step 1's MFMAs.
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) {
        dma_head(kt0 + i);
        dma_tail(kt0 + i);
      }
      dma_head(kt0 + NS - 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * ROUNDS + H, 15));
      __builtin_amdgcn_s_barrier();
      Frags F0, F1;
      read_step(kt0, 0, F0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      for (int kt = kt0; kt < kt1; ++kt) {
        read_step(kt, 1, F1);
        dma_tail(kt + NS - 1);
        mfmas(F0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::IN_FLIGHT, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma_head(kt + NS);
        read_step(kt + 1, 0, F0);
        mfmas(F1);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    }
  } else {
    if (kt0 < kt1) {
      // Each group takes its own step of every stage: the tail of stage
      // kt+NS-1's DMA with the first two MFMAs; wait for stage kt+1 (kt+2
      // with the A expansion's lookahead) and sync; the head of stage
      // kt+NS's DMA, the expansion of stage kt+2's A and the reads of stage
      // kt+1 with the last two.  A buffer kt % 2 is free then: its reads (of
      // stage kt) were done before the sync.
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) {
        dma_head(kt0 + i);
        dma_tail(kt0 + i);
      }
      dma_head(kt0 + NS - 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - (C::AEXP ? 3 : 2)) * ROUNDS + H, 15));
      __builtin_amdgcn_s_barrier();
      if constexpr (C::AEXP) {
        expand_a(kt0);
        expand_a(kt0 + 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        __builtin_amdgcn_s_barrier();
      }
      Frags F0, F1;
      read_step(kt0, kg, F0);
      auto stage = [&](int kt, const Frags& f, Frags& g) __attribute__((always_inline)) {
        dma_tail(kt + NS - 1);
        mfmas(f, 0, 2);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::IN_FLIGHT, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma_head(kt + NS);
        expand_a(kt + 2);
        read_step(kt + 1, kg, g);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(f, 2, 4);
        __builtin_amdgcn_sched_barrier(0);
      };
      int kt = kt0;
      for (; kt + 1 < kt1; kt += 2) {
        stage(kt, F0, F1);
        stage(kt + 1, F1, F0);
      }
      if (kt < kt1) stage(kt, F0, F1);
    }
    // Sum of the two groups through LDS (every wave has passed its last
    // read; the DMAs still in flight land in ring slots, so wait for them),
    // lane-contiguous dwords.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    float* red = reinterpret_cast<float*>(dyn_lds) + wg * TM * TN * 1024;
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) red[((i * TN + j) * 16 + e) * 64 + lane] = acc[i][j][e];
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    __builtin_amdgcn_s_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += red[((i * TN + j) * 16 + e) * 64 + lane];
  }

  const float g = (PARTIAL || C::MX) ? 1.0f : (*ags) * (*bgs);
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (full || (row < M && col < N)) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e] * g);
        }
        if (e == 15) __builtin_amdgcn_sched_barrier(0);
      }
}

// ------------------------------------------------------------------ W4A16
// Weight-only FP4: Y[M, N] = A[M, K] (bf16) * dequant(B)[N, K]^T with fp32
// accumulation on v_mfma_f32_32x32x16_bf16 ("Bridging the Gap ...": the
// W4A16 control of the FP4 weight formats; decode streams the weights).
//
// One ring carries both operands: per K-stage of 128, the BM activation rows
// (256 bytes of bf16 each), the BN weight rows' codes (64 bytes each) and
// their scales stream into an NS-slot LDS ring by DMA, as in the FP4 kernels.
// Eight waves: wave w takes 64-K step w / 4 of every stage, and the four
// waves of a step share the BM x 128 output tile.  With WMS = 1 each owns all
// BM rows and 32 weight columns, so every weight fragment is expanded to bf16
// once per workgroup (MXFP4: the hardware decode applies the E8M0 scale
// exactly; NVFP4: e2m1 * e4m3 in fp32, exact in bf16) and feeds BM / 32
// MFMAs.  With WMS = 2 each owns BM / 2 rows and 64 columns: the weights are
// expanded twice, but each activation fragment read from LDS feeds two MFMAs
// instead of one (the cheaper trade where expansion is cheap, MXFP4).  Two
// waves per SIMD hide each other's LDS reads and expansion; the two step
// groups' accumulators are summed through LDS at the end.  B's K order within a 64-K step is the FP4
// kernels' (lane half h, dword t of its 32 codes); A's lane reads the same K
// positions, chunk 8s + 4h + t of its row.  A rows rotate their sixteen
// 16-byte chunks by row % 16, so the sixteen rows a fragment read serves at
// once hit sixteen different bank groups; NVFP4 scales are read as one
// 16-byte piece per row (sixteen consecutive rows: one bank line) rather
// than as 16-bit loads at a 16-byte stride.
template <int FMT, int BM, int NS, int WMS>
struct W4Cfg {
  static constexpr int BN = 128, NW = 8, WM = BM / WMS, WN = 32 * WMS;
  static constexpr int TM = WM / 32, TN = WN / 32, NWN = BN / WN;
  static_assert(TM >= 1 && NWN * WMS == 4, "four waves per step cover the tile");
  static constexpr int B_CODES = BM * 256;  // A: BM rows x 128 bf16
  static constexpr int B_SC = B_CODES + BN * 64;
  static constexpr int USED = B_SC + (fmt_mx(FMT) ? (BN / 32) * 256 : BN * 16);
  static constexpr int SC_ADV = fmt_mx(FMT) ? 256 : 16;  // scale bytes per 256-K chunk and source
  static constexpr int RB = NW * 1024;
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  static constexpr int LDS = NS * STAGE;
  static constexpr int IN_FLIGHT = (NS - 2) * ROUNDS;
  static_assert(B_CODES % RB == 0 && (BN * 64) % RB == 0, "rounds hold one kind of data");
  static_assert(NS >= 3 && (NS - 1) * ROUNDS <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Eight E2M1 codes -> eight bf16 times 2^E (E8M0 scale as the operand's exponent).
__device__ __forceinline__ u32x4 expand8_bf16_mx(uint32_t w, float scale) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
}

// Eight E2M1 codes times an E4M3 value.  Each product has at most six
// significant bits and lies in [2^-10, 2688], so its fp32 form has sixteen
// zero low bits and the bf16 value is the high half, taken without rounding.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
}
__device__ __forceinline__ u32x4 expand8_bf16_nv(uint32_t w, float s) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  return u32x4{pack_bf16(v0[0] * s, v0[1] * s), pack_bf16(v1[0] * s, v1[1] * s),
               pack_bf16(v2[0] * s, v2[1] * s), pack_bf16(v3[0] * s, v3[1] * s)};
}

template <int TM, int TN, bool MX>
struct W4Frags {
  u32x4 a[TM][4];  // A: four chunks (one per MFMA of the step) per 32-row fragment
  u32x4 b[TN];     // 32 weight columns each: 32 codes per lane
  // raw scale words, decoded in the MFMA phase (decoding them on arrival
  // would wait for every LDS read issued before them): MX the lane's scale
  // dword of the tile (one byte per 64-K step), NV the row's 16 E4M3 bytes
  std::conditional_t<MX, uint32_t, u32x4> sc[TN];
};

template <int FMT, int BM, int NS, int WMS, int YDT, bool PARTIAL>
__global__ __launch_bounds__(512) void gemm_w4a16_kernel(
    const uint8_t* __restrict__ A, int64_t lda_bytes, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ bgs, void* __restrict__ Y,
    int64_t ldy, int M, int N, int K, int kchunks, int tiles_n, int kt_per_split,
    float* __restrict__ part, int bt) {
  using C = W4Cfg<FMT, BM, NS, WMS>;
  constexpr int TM = C::TM, TN = C::TN, BN = C::BN, ROUNDS = C::ROUNDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave >> 2;  // the 64-K step of each stage this wave takes
  const int wn = (wave & 3) % C::NWN, wm = (wave & 3) / C::NWN;
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // DMA sources of this thread, one per round: A rows, B code rows, then the
  // scale pieces of the stage (and slot padding, which re-reads scales).
  const uint8_t* src[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (r * C::RB < C::B_CODES) {
      const int row = p >> 8, chunk = ((p >> 4) & 15) ^ (row & 15);
      src[r] = A + (int64_t)min(m0 + row, M - 1) * lda_bytes + chunk * 16;
    } else if (r * C::RB < C::B_SC) {
      const int row = (p - C::B_CODES) >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + code_offset(min(n0 + row, N - 1), chunk * 16, rowbytes, bt != 0);
    } else if (p < C::USED) {
      const int q = p - C::B_SC;
      if constexpr (fmt_mx(FMT))
        src[r] = Bs + (int64_t)min((n0 >> 5) + (q >> 8), (N - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = Bs + (int64_t)min(n0 + (q >> 4), N - 1) * (K / 16);
    } else {
      src[r] = Bs;
    }
  }
  auto slot_of = [&](int kt) __attribute__((always_inline)) {
    return dyn_lds + (kt % NS) * C::STAGE;
  };
  constexpr int H = ROUNDS / 2;
  const int64_t badv = bt ? 8192 : 64;  // tiled B codes: the next 8 KB tile
  auto dma = [&](int kt, int r) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
    const int64_t adv = r * C::RB < C::B_CODES ? (int64_t)ks * 256
                        : r * C::RB < C::B_SC  ? (int64_t)ks * badv
                                               : (int64_t)(ks >> 1) * C::SC_ADV;
    dma16(src[r] + adv, slot_of(kt) + r * C::RB + wave * 1024);
  };
  auto dma_head = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < H; ++r) dma(kt, r);
  };
  auto dma_tail = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int r = H; r < ROUNDS; ++r) dma(kt, r);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  using Frags = W4Frags<TM, TN, fmt_mx(FMT)>;
  // the weights' pieces first: the expansion that opens the MFMA phase needs
  // them before any activation fragment
  auto read_step = [&](int kt, int s, Frags& f) __attribute__((always_inline)) {
    const uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int brow = wn * C::WN + j * 32 + (lane & 31);  // the lane's weight row in the tile
      f.b[j] = *reinterpret_cast<const u32x4*>(slot + C::B_CODES + brow * 64 +
                                               (((2 * s + h) ^ swz4(brow)) * 16));
      if constexpr (fmt_mx(FMT))
        f.sc[j] = *reinterpret_cast<const uint32_t*>(slot + C::B_SC + (brow >> 5) * 256 +
                                                     (lane & 31) * 4 + h * 128);
      else
        f.sc[j] = *reinterpret_cast<const u32x4*>(slot + C::B_SC + brow * 16);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint8_t* ar = slot + (wm * C::WM + i * 32 + (lane & 31)) * 256;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        f.a[i][t] = *reinterpret_cast<const u32x4*>(ar + (((8 * s + 4 * h + t) ^ (lane & 15)) * 16));
    }
  };
  // MFMAs t0 .. t1-1 of the step s of stage kt (one per 16-K piece of the
  // lane's codes)
  auto mfmas = [&](int kt, int s, const Frags& f, int t0, int t1) __attribute__((always_inline)) {
    float s0[TN], s1[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (fmt_mx(FMT)) {
        const uint32_t code = (f.sc[j] >> (8 * (2 * (kt & 1) + s))) & 0xFFu;
        s0[j] = s1[j] = fmt_int(FMT) ? e8m0_value(code) : e8m0_as_cvt_scale(code);
      } else {
        const uint32_t lo = (kt & 1) ? f.sc[j][2] : f.sc[j][0], hi = (kt & 1) ? f.sc[j][3] : f.sc[j][1];
        const uint32_t w = (s ? hi : lo) >> (16 * h);
        const f32x2 sv = e4m3x2_f32(w);
        s0[j] = sv[0];
        s1[j] = sv[1];
      }
    }
#pragma unroll
    for (int t = t0; t < t1; ++t) {
      u32x4 bv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float sc = t < 2 ? s0[j] : s1[j];
        if constexpr (fmt_int(FMT))
          bv[j] = expand8_i4_bf16(f.b[j][t], sc);
        else if constexpr (fmt_mx(FMT))
          bv[j] = expand8_bf16_mx(f.b[j][t], sc);
        else
          bv[j] = expand8_bf16_nv(f.b[j][t], sc);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16(f.a[i][t], bv[j], acc[i][j]);
    }
  };

  if (kt0 < kt1) {
    // Per stage (this wave's step of it, fragments already in registers):
    // the tail of stage kt+NS-1's DMA with the first two MFMAs; wait for
    // stage kt+1 and sync; the head of stage kt+NS's DMA (into slot kt, which
    // nobody reads after the sync) and the reads of stage kt+1 with the last
    // two MFMAs, so the reads' latency falls under MFMA work although all
    // waves leave the barrier together.
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) {
      dma_head(kt0 + i);
      dma_tail(kt0 + i);
    }
    dma_head(kt0 + NS - 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * ROUNDS + H, 15));
    __builtin_amdgcn_s_barrier();
    Frags F0, F1;
    read_step(kt0, kg, F0);
    auto stage = [&](int kt, const Frags& f, Frags& g) __attribute__((always_inline)) {
      dma_tail(kt + NS - 1);
      mfmas(kt, kg, f, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::IN_FLIGHT, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      dma_head(kt + NS);
      read_step(kt + 1, kg, g);
      __builtin_amdgcn_sched_barrier(0);  // the reads go out before the MFMAs
      mfmas(kt, kg, f, 2, 4);
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = kt0;
    for (; kt + 1 < kt1; kt += 2) {
      stage(kt, F0, F1);
      stage(kt + 1, F1, F0);
    }
    if (kt < kt1) stage(kt, F0, F1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  }

  // Sum of the two step groups: the second group's accumulators go through
  // LDS (the ring is idle: every wave has passed its last read and waited for
  // its DMAs), lane-contiguous dwords.
  static_assert(4 * TM * TN * 4096 <= C::LDS, "reduction fits the ring");
  float* red = reinterpret_cast<float*>(dyn_lds) + (wave & 3) * TM * TN * 1024;
  __builtin_amdgcn_s_barrier();
  if (kg == 1) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[((i * TN + j) * 16 + e) * 64 + lane] = acc[i][j][e];
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  if (kg == 1) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] += red[((i * TN + j) * 16 + e) * 64 + lane];

  const float g = (!fmt_mx(FMT) && !PARTIAL) ? *bgs : 1.0f;
  const bool full = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * C::WM + i * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
        const int col = n0 + wn * C::WN + j * 32 + (lane & 31);
        if (full || (row < M && col < N)) {
          if constexpr (PARTIAL)
            part[((int64_t)blockIdx.y * M + row) * N + col] = acc[i][j][e];
          else
            store_out<YDT>(Y, ldy, row, col, acc[i][j][e] * g);
        }
        if (e == 15) __builtin_amdgcn_sched_barrier(0);
      }
}

// The ring needs more than the default 64 KB of LDS; raise the limit once.
template <int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL>
hipError_t mx_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_mx_kernel<BM, BN, WM, WN, NS, YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, MxCfg<BM, BN, WM, WN, NS>::LDS);
  return status;
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_mx_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                         const uint8_t* b, const uint8_t* bs, int bt, void* y, int ydt, int64_t ldy,
                         int splits, int kt_per, float* part, hipStream_t st) {
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  const int kchunks = (int)mx_gemm_kchunks(K);
  const size_t lds = MxCfg<BM, BN, WM, WN, NS>::LDS;
  hipError_t e;
  if (splits > 1) {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_F32, true><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  } else if (ydt == FP4_DT_F32) {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_F32, false><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  } else {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_BF16, false>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_BF16, false><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int YDT, bool PARTIAL>
hipError_t mx2_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_mx2_kernel<BM, BN, WM, WN, YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Mx2Cfg<BM, BN, WM, WN>::LDS);
  return status;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_mx2_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const uint8_t* b, const uint8_t* bs, int bt, void* y, int ydt, int64_t ldy,
                          int splits, int ks_per, float* part, hipStream_t st) {
  using C = Mx2Cfg<BM, BN, WM, WN>;
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  const int kchunks = (int)mx_gemm_kchunks(K);
  hipError_t e;
  if (splits > 1) {
    if ((e = mx2_lds_attr<BM, BN, WM, WN, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_mx2_kernel<BM, BN, WM, WN, FP4_DT_F32, true><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, ks_per, part, 0, bt);
  } else if (ydt == FP4_DT_F32) {
    if ((e = mx2_lds_attr<BM, BN, WM, WN, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_mx2_kernel<BM, BN, WM, WN, FP4_DT_F32, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, ks_per, part, 0, bt);
  } else {
    if ((e = mx2_lds_attr<BM, BN, WM, WN, FP4_DT_BF16, false>()) != hipSuccess) return e;
    const int vec_out = (ldy % 8 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15u) == 0);
    gemm_mx2_kernel<BM, BN, WM, WN, FP4_DT_BF16, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, ks_per, part, vec_out, bt);
  }
  return hipGetLastError();
}

template <int FMT, int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL, int KG>
hipError_t nv_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, YDT, PARTIAL, KG>),
      hipFuncAttributeMaxDynamicSharedMemorySize, NvCfg<BM, BN, WM, WN, NS, FMT, KG>::LDS);
  return status;
}

template <int BM, int BN, int WM, int WN, int NS, int FMT = FP4_FMT_NVFP4, int KG = 1>
hipError_t launch_nv_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                         const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                         int bt, void* y, int ydt, int64_t ldy, int splits, int kt_per, float* part,
                         hipStream_t st) {
  using C = NvCfg<BM, BN, WM, WN, NS, FMT, KG>;
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  hipError_t e;
  if (splits > 1) {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, true, KG>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, true, KG><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part, bt);
  } else if (ydt == FP4_DT_F32) {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, false, KG>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, false, KG><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part, bt);
  } else {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_BF16, false, KG>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_BF16, false, KG><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part, bt);
  }
  return hipGetLastError();
}

template <int FMT, int BM, int NS, int WMS, int YDT, bool PARTIAL>
hipError_t w4_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_w4a16_kernel<FMT, BM, NS, WMS, YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, W4Cfg<FMT, BM, NS, WMS>::LDS);
  return status;
}

template <int FMT, int BM, int NS, int WMS>
hipError_t launch_w4_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda_bytes,
                         const uint8_t* b, const uint8_t* bs, const float* bgs, int bt, void* y, int ydt,
                         int64_t ldy, int splits, int kt_per, float* part, hipStream_t st) {
  using C = W4Cfg<FMT, BM, NS, WMS>;
  const int tiles_n = (int)((N + C::BN - 1) / C::BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  const int kchunks = (int)mx_gemm_kchunks(K);
  hipError_t e;
  if (splits > 1) {
    if ((e = w4_lds_attr<FMT, BM, NS, WMS, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, BM, NS, WMS, FP4_DT_F32, true><<<grid, C::NW * 64, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  } else if (ydt == FP4_DT_F32) {
    if ((e = w4_lds_attr<FMT, BM, NS, WMS, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, BM, NS, WMS, FP4_DT_F32, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  } else {
    if ((e = w4_lds_attr<FMT, BM, NS, WMS, FP4_DT_BF16, false>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, BM, NS, WMS, FP4_DT_BF16, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part, bt);
  }
  return hipGetLastError();
}

// Row tile of the weight-only GEMM: the rows of M up to 128 in one tile (32,
// 64 or 128; shallower tiles get deeper rings), 128 weight columns.  Split K
// while fewer than 256 workgroups would run (at least 4 stages per slice,
// slices of whole 256-K scale chunks).
struct W4Plan {
  int bm, splits, kt_per;
};
W4Plan plan_w4(int64_t M, int64_t N, int64_t K) {
  const int bm = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + 127) / 128);
  const int KT = (int)(K / 128);
  int splits = 1;
  while (tiles * splits * 2 <= 256 && splits < kMaxSplits && KT / (splits * 2) >= 4) splits *= 2;
  int kt_per = (KT + splits - 1) / splits;
  kt_per += kt_per & 1;
  return W4Plan{bm, splits, kt_per};
}

template <int FMT>
hipError_t launch_w4_fmt(int bm, int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda_bytes,
                         const uint8_t* b, const uint8_t* bs, const float* bgs, int bt, void* y, int ydt,
                         int64_t ldy, int splits, int kt_per, float* part, hipStream_t st) {
  // MXFP4 expands cheaply: split the rows over two waves to halve the
  // activation reads; the other formats expand each weight fragment once.
  constexpr int WMS = FMT == FP4_FMT_MXFP4 ? 2 : 1;
  if (bm == 32)
    return launch_w4_cfg<FMT, 32, 6, 1>(M, N, K, a, lda_bytes, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  if (bm == 64)
    return launch_w4_cfg<FMT, 64, 4, WMS>(M, N, K, a, lda_bytes, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  return launch_w4_cfg<FMT, 128, 3, WMS>(M, N, K, a, lda_bytes, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
}

// Y = 0 (a product over an empty K range).
__global__ __launch_bounds__(kThreads) void zero_out_kernel(void* __restrict__ Y, int ydt, int M,
                                                            int N, int64_t ldy) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int row = (int)(i / N), col = (int)(i - (int64_t)row * N);
    if (ydt == FP4_DT_F32) store_out<FP4_DT_F32>(Y, ldy, row, col, 0.0f);
    else store_out<FP4_DT_BF16>(Y, ldy, row, col, 0.0f);
  }
}

// Y = sum over splits of the fp32 partials (fixed order), times the tensor
// scales that are given (NVFP4: (*ga) * (*gb); weight-only NVFP4: *ga).
template <int YDT, bool VEC>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 int splits, int M, int N,
                                                                 void* __restrict__ Y,
                                                                 int64_t ldy,
                                                                 const float* __restrict__ ga,
                                                                 const float* __restrict__ gb) {
  const int64_t total = (int64_t)M * N;
  const bool scaled = ga != nullptr || gb != nullptr;
  const float g = (ga ? *ga : 1.0f) * (gb ? *gb : 1.0f);
  if constexpr (VEC) {
    // four consecutive outputs (one row, N % 4 == 0) per thread; all of its
    // 16-byte partial loads go out before the sums, which keep slice order
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total / 4;
         v += (int64_t)gridDim.x * kThreads) {
      f32x4 p[kMaxSplits];
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k)
        if (k < splits) p[k] = *reinterpret_cast<const f32x4*>(part + (int64_t)k * total + 4 * v);
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k)
        if (k < splits) acc += p[k];
      const int row = (int)((4 * v) / N), col = (int)(4 * v - (int64_t)row * N);
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out<YDT>(Y, ldy, row, col + e, scaled ? acc[e] * g : acc[e]);
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
      float acc = 0.0f;
      for (int k = 0; k < splits; ++k) acc += part[(int64_t)k * total + i];
      const int row = (int)(i / N), col = (int)(i - (int64_t)row * N);
      store_out<YDT>(Y, ldy, row, col, scaled ? acc * g : acc);
    }
  }
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, void* y,
                                int ydt, int64_t ldy, const float* ga, const float* gb,
                                hipStream_t st) {
  const bool vec = N % 4 == 0 && splits <= kMaxSplits;
  int64_t g = (M * N / (vec ? 4 : 1) + kThreads - 1) / kThreads;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  if (ydt == FP4_DT_F32 && vec)
    splitk_reduce_kernel<FP4_DT_F32, true><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
  else if (ydt == FP4_DT_F32)
    splitk_reduce_kernel<FP4_DT_F32, false><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
  else if (vec)
    splitk_reduce_kernel<FP4_DT_BF16, true><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
  else
    splitk_reduce_kernel<FP4_DT_BF16, false><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ NVFP4
// Block tile 128 x 128, K-stage of 64 (4 NVFP4 blocks), four waves of 64 x 64
// built from 16x16x32 fp16 MFMA tiles.  Each thread dequantizes one 16-byte
// chunk (32 elements, two blocks) of A and one of B per stage into LDS.
template <int YDT>
__global__ __launch_bounds__(kThreads) void gemm_nv_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ ags,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ bgs,
    void* __restrict__ Y, int64_t ldy, int M, int N, int K, int tiles_n, int bt) {
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
    rb = *reinterpret_cast<const u32x4*>(B + code_offset(b_row, (int64_t)kt * 32 + c_half * 16, rowbytes, bt != 0));
    sca = *reinterpret_cast<const uint16_t*>(As + (int64_t)a_row * srow + kt * 4 + c_half * 2);
    scb = *reinterpret_cast<const uint16_t*>(Bs + (int64_t)b_row * srow + kt * 4 + c_half * 2);
  };
  // 16 bytes of codes + two E4M3 scale bytes -> 32 fp16 values -> 4 LDS chunks.
  auto expand = [&](u32x4 codes, uint32_t sc2, uint8_t* dst_row) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const _Float16 s = e4m3x2_f16(sc2)[blk];
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
  int cfg;     // 0: 256x256, 8 waves (large M and N), 1: 128x128, 2: 32 x bn2 (M <= 32)
  int splits;  // split-K factor (1 = none)
  int kt_per;  // K-stages per split (even: slices start on a 256-K scale chunk)
};

// bn2: width of the M <= 32 tiles (MXFP4 128: measured 5-10 % faster at
// decode than 256 with a 6-stage ring; the NVFP4 ring keeps 256).  small_m_cap:
// also stop the 128x128 tiles at 256 workgroups when M <= 128 (MXFP4: at
// M = 128 the weights stream 20-25 % faster without the extra slices).
MxPlan plan_mx(int64_t M, int64_t N, int64_t K, int bn2 = 256, bool small_m_cap = false) {
  MxPlan p{1, 1, (int)(K / 128)};
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (M <= 32) p.cfg = 2;
  else if (big_tiles >= 256) p.cfg = 0;
  else p.cfg = 1;
  const int bm = p.cfg == 0 ? 256 : (p.cfg == 1 ? 128 : 32);
  const int bn = p.cfg == 1 ? 128 : (p.cfg == 2 ? bn2 : 256);
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int KT = (int)(K / 128);
  // Split K while fewer than 512 workgroups (two per CU) would run, keeping
  // at least 4 stages per slice.  Only for tiles that leave the chip idle.
  // The 32-row decode tiles stop at 256 workgroups: measured with four
  // rotating 117 MB weight copies, 224 / 256 workgroups stream the weights
  // 7-8 % faster than 448 / 512 (fewer slices, less partial traffic).
  int splits = 1;
  const int64_t cap = (p.cfg == 2 || (small_m_cap && p.cfg == 1 && M <= 128)) ? 256 : 512;
  if (p.cfg != 0)
    while (tiles * splits * 2 <= cap && splits < kMaxSplits && KT / (splits * 2) >= 4) splits *= 2;
  p.splits = splits;
  p.kt_per = (KT + splits - 1) / splits;
  p.kt_per += p.kt_per & 1;
  return p;
}

}  // namespace

namespace fp4lib {

// The MXFP4 plan: plan_mx, except that 128 x 128 tiles above 128 rows with
// K % 256 == 0 (and 32-bit DMA offsets) run unsplit on the 256-K kernel with
// eight waves of 64 x 32.  Measured against the split plan on the 128-K ring
// with its fp32 partials and reduction (side by side, bf16 output):
// 1024x4096x4096 31.9 -> 17.7 us, 384x4096x4096 24.5 -> 13.8,
// 2048x1024x2048 26.9 -> 8.7, and faster at every tile count down to 16
// (256x1024x8192 19.3 -> 18.6 us).
bool mx_unsplit_128(int64_t M, int64_t N, int64_t K) {
  return M > 128 && K % 256 == 0 && (uint64_t)max(M, N) * (uint64_t)(K / 2) < (1ull << 32);
}

MxPlan plan_mx_fp4(int64_t M, int64_t N, int64_t K) {
  MxPlan p = plan_mx(M, N, K, 128, true);
  if (p.cfg == 1 && mx_unsplit_128(M, N, K)) {
    p.splits = 1;
    p.kt_per = (int)(K / 128);
  }
  return p;
}

size_t gemm_mx_workspace(int64_t M, int64_t N, int64_t K) {
  MxPlan p = plan_mx_fp4(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const uint8_t* b, const uint8_t* bs, int bt, void* y, int ydt, int64_t ldy,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {  // empty sum
    zero_out_kernel<<<256, kThreads, 0, st>>>(y, ydt, (int)M, (int)N, ldy);
    return hipGetLastError();
  }
  MxPlan p = plan_mx_fp4(M, N, K);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_mx_workspace(M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  // 256 x 256 tiles: K-stages of 256 (whole 128-byte lines per row and DMA,
  // measured 2-13 % faster on the Llama shapes than the 128-K ring) when K
  // allows them
  // (its DMA offsets are 32-bit: operands under 4 GB)
  if (p.cfg == 0 && K % 256 == 0 && splits == 1 && (uint64_t)max(M, N) * (uint64_t)(K / 2) < (1ull << 32))
    e = launch_mx2_cfg<256, 256, 128, 64>(M, N, K, a, as, b, bs, bt, y, ydt, ldy, 1, (int)(K / 256), part, st);
  else if (p.cfg == 0)
    e = launch_mx_cfg<256, 256, 128, 64, 4>(M, N, K, a, as, b, bs, bt, y, ydt, ldy, splits, kt_per, part, st);
  // 128 x 128 tiles above 128 rows (plan_mx_fp4: unsplit): the 256-K kernel
  // with eight waves of 64 x 32 (2048x4096x4096 32.6 -> 26.6 us,
  // 512x14336x4096 30.5 -> 24.8 us against the 128-K ring; slower at 64-96
  // rows, level at 128)
  else if (p.cfg == 1 && mx_unsplit_128(M, N, K))
    e = launch_mx2_cfg<128, 128, 64, 32>(M, N, K, a, as, b, bs, bt, y, ydt, ldy, 1, (int)(K / 256), part, st);
  else if (p.cfg == 1)
    e = launch_mx_cfg<128, 128, 64, 64, 4>(M, N, K, a, as, b, bs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_mx_cfg<32, 128, 32, 32, 6>(M, N, K, a, as, b, bs, bt, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, nullptr, nullptr, st);
}

// The NVFP4 / INT4 ring plans: as MXFP4's, and at M <= 128 the 128x128
// tiles run two K-step groups of waves and stop at 256 workgroups (K8192
// N28672, M = 128: 95 -> 83 us against one group with split-K 2; at M >= 256
// one group stays faster).  NVFP4 waves there own 64x64 sub-tiles; the INT4
// formats, whose expansion costs more, own all 128 rows x 32 columns with
// the A tile expanded once per workgroup into LDS (NVINT4 128 -> 109 us,
// MXINT4 155 -> 127 us; NVFP4 80 -> 95 us that way, so it keeps 64x64).
// The ring GEMMs' plan for format fmt (NVFP4, MXINT4, NVINT4): plan_mx,
// except that NVFP4 above 128 rows with at least 128 tiles of 128 x 128 runs
// unsplit.  Measured against split-K plus the reduction kernel (side by
// side, bf16 output): 1024x4096x4096 55.1 -> 48.3 us, 2048x1024x2048 32.1 ->
// 23.4 us; with fewer tiles the split plan is faster (256x1024x8192, 16
// tiles: 22.6 against 67.4 us unsplit).  (MXINT4 lost 9 % on 2048x1024x2048
// unsplit, NVINT4 gained 3-5 %: both keep the split plan.)
MxPlan plan_nv(int fmt, int64_t M, int64_t N, int64_t K) {
  MxPlan p = plan_mx(M, N, K, 256, true);
  if (fmt == FP4_FMT_NVFP4 && p.cfg == 1 && M > 128 && ((M + 127) / 128) * ((N + 127) / 128) >= 128) {
    p.splits = 1;
    p.kt_per = (int)(K / 128);
  }
  return p;
}

size_t gemm_nv_workspace(int fmt, int64_t M, int64_t N, int64_t K) {
  if (K % 256 != 0 || K == 0) return 0;
  MxPlan p = plan_nv(fmt, M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// The ring GEMM with expanded operands for INT4 elements: NVINT4 on fp16
// MFMA (n * e4m3 exact in fp16), MXINT4 on bf16 MFMA (n * 2^e exact in bf16).
template <int FMT>
hipError_t launch_ring_int4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                            const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                            int bt, void* y, int ydt, int64_t ldy, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  MxPlan p = plan_nv(FMT, M, N, K);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_nv_workspace(FMT, M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  if (p.cfg == 0)
    e = launch_nv_cfg<256, 256, 128, 128, 3, FMT>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else if (p.cfg == 1 && M <= 128)
    e = launch_nv_cfg<128, 128, 128, 32, 4, FMT, 2>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else if (p.cfg == 1)
    e = launch_nv_cfg<128, 128, 64, 64, 3, FMT>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_nv_cfg<32, 256, 32, 64, 4, FMT, 2>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, fmt_mx(FMT) ? nullptr : ags,
                              fmt_mx(FMT) ? nullptr : bgs, st);
}

hipError_t launch_gemm_int4(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                            const uint8_t* as, const float* ags, const uint8_t* b, const uint8_t* bs,
                            const float* bgs, int bt, void* y, int ydt, int64_t ldy, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    zero_out_kernel<<<256, kThreads, 0, st>>>(y, ydt, (int)M, (int)N, ldy);
    return hipGetLastError();
  }
  if (fmt == FP4_FMT_MXINT4)
    return launch_ring_int4<FP4_FMT_MXINT4>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, ws, ws_bytes, st);
  return launch_ring_int4<FP4_FMT_NVINT4>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, ws, ws_bytes, st);
}

hipError_t launch_gemm_nv(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                          int bt, void* y, int ydt, int64_t ldy, void* ws, size_t ws_bytes,
                          hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 256 == 0 && K > 0) {
    // LDS ring with in-register fp16 expansion; tiles and split-K as for MXFP4
    MxPlan p = plan_nv(FP4_FMT_NVFP4, M, N, K);
    const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_nv_workspace(FP4_FMT_NVFP4, M, N, K);
    const int splits = split ? p.splits : 1;
    const int kt_per = split ? p.kt_per : (int)(K / 128);
    float* part = static_cast<float*>(ws);
    hipError_t e;
    if (p.cfg == 0)  // eight waves of 128x64 (two per SIMD): 4096^3 133 -> 126 us, 70B shapes level
      e = launch_nv_cfg<256, 256, 128, 64, 3>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
    else if (p.cfg == 1 && M <= 128)
      e = launch_nv_cfg<128, 128, 64, 64, 3, FP4_FMT_NVFP4, 2>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
    else if (p.cfg == 1)
      e = launch_nv_cfg<128, 128, 64, 64, 3>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
    else  // M <= 32: two K-step groups of four waves (two waves per SIMD)
      e = launch_nv_cfg<32, 256, 32, 64, 4, FP4_FMT_NVFP4, 2>(M, N, K, a, as, ags, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
    if (e != hipSuccess || !split) return e;
    return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, ags, bgs, st);
  }
  const int tiles_n = (int)((N + 127) / 128);
  const unsigned grid = (unsigned)(((M + 127) / 128) * tiles_n);
  if (ydt == FP4_DT_F32)
    gemm_nv_kernel<FP4_DT_F32><<<grid, kThreads, 0, st>>>(a, as, ags, b, bs, bgs, y, ldy, (int)M,
                                                          (int)N, (int)K, tiles_n, bt);
  else
    gemm_nv_kernel<FP4_DT_BF16><<<grid, kThreads, 0, st>>>(a, as, ags, b, bs, bgs, y, ldy, (int)M,
                                                           (int)N, (int)K, tiles_n, bt);
  return hipGetLastError();
}

size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K) {
  if (K % 256 != 0 || K == 0 || M == 0 || N == 0) return 0;
  W4Plan p = plan_w4(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_w4a16(int fmt, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                             const uint8_t* b, const uint8_t* bs, const float* bgs, int bt, void* y,
                             int ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    zero_out_kernel<<<256, kThreads, 0, st>>>(y, ydt, (int)M, (int)N, ldy);
    return hipGetLastError();
  }
  W4Plan p = plan_w4(M, N, K);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_w4a16_workspace(M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
  const uint8_t* ab = static_cast<const uint8_t*>(a);
  hipError_t e;
  if (fmt == FP4_FMT_MXFP4)
    e = launch_w4_fmt<FP4_FMT_MXFP4>(p.bm, M, N, K, ab, lda * 2, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else if (fmt == FP4_FMT_NVFP4)
    e = launch_w4_fmt<FP4_FMT_NVFP4>(p.bm, M, N, K, ab, lda * 2, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else if (fmt == FP4_FMT_MXINT4)
    e = launch_w4_fmt<FP4_FMT_MXINT4>(p.bm, M, N, K, ab, lda * 2, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_w4_fmt<FP4_FMT_NVINT4>(p.bm, M, N, K, ab, lda * 2, b, bs, bgs, bt, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy,
                              fmt_mx(fmt) ? nullptr : bgs, nullptr, st);
}

}  // namespace fp4lib
