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
#include <type_traits>

#include "fp4_device.h"
#include "launch.h"

using namespace fp4k;

namespace {

constexpr int kThreads = 256;

// XOR swizzle of 16-byte chunks within a 64-byte LDS row (4 chunks): four
// consecutive rows share a 256-byte bank line, so rows 4i .. 4i+3 keep their
// chunk order and each group of four rows rotates it by i.  The fragment reads
// (lane l: row l % 32, one chunk) then see no bank conflicts (measured with
// SQ_LDS_BANK_CONFLICT on gfx950; a rotation by bits 1-2 of the row was 2-way).
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }
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

// gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; a field at its maximum does not wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

template <int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL>
__global__ __launch_bounds__((MxCfg<BM, BN, WM, WN, NS>::NW * 64)) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, void* __restrict__ Y, int64_t ldy, int M, int N, int K,
    int kchunks, int tiles_n, int kt_per_split, float* __restrict__ part) {
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

  // DMA sources of this thread, one per round: slot byte p = r*RB + tid*16.
  const uint8_t* src[ROUNDS];
  bool code_src[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < C::B_CODES) {
      const int row = p >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = A + (int64_t)min(m0 + row, M - 1) * rowbytes + chunk * 16;
      code_src[r] = true;
    } else if (p < C::A_SC) {
      const int row = (p - C::B_CODES) >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + (int64_t)min(n0 + row, N - 1) * rowbytes + chunk * 16;
      code_src[r] = true;
    } else if (p < C::B_SC) {
      const int t = (p - C::A_SC) >> 8;
      src[r] = As + (int64_t)min((m0 >> 5) + t, (M - 1) >> 5) * kchunks * 256 + (p & 255);
      code_src[r] = false;
    } else if (p < C::USED) {
      const int t = (p - C::B_SC) >> 8;
      src[r] = Bs + (int64_t)min((n0 >> 5) + t, (N - 1) >> 5) * kchunks * 256 + (p & 255);
      code_src[r] = false;
    } else {  // slot padding: any valid address
      src[r] = As + (p & 255);
      code_src[r] = false;
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
      dma16(src[r] + (code_src[r] ? ks * 64 : (ks >> 1) * 256), slot + r * C::RB + wave * 1024);
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
      dma16(src[r] + (code_src[r] ? ks * 64 : (ks >> 1) * 256), slot + r * C::RB + wave * 1024);
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
template <int BM, int BN, int WM, int WN, int NS, int FMT = FP4_FMT_NVFP4>
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
  static constexpr int NW = (BM / WM) * (BN / WN);
  static constexpr int RB = NW * 1024;
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  static constexpr int LDS = NS * STAGE;
  static constexpr int IN_FLIGHT = (NS - 2) * ROUNDS;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NS >= 3 && (NS - 1) * ROUNDS <= 63, "vmcnt range");
};

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
};

template <int FMT, int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL>
__global__ __launch_bounds__((NvCfg<BM, BN, WM, WN, NS, FMT>::NW * 64)) void gemm_nv_ring_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const float* __restrict__ ags,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const float* __restrict__ bgs,
    void* __restrict__ Y, int64_t ldy, int M, int N, int K, int tiles_n, int kt_per_split,
    float* __restrict__ part) {
  using C = NvCfg<BM, BN, WM, WN, NS, FMT>;
  constexpr int TM = C::TM, TN = C::TN, ROUNDS = C::ROUNDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / (BN / WN), wn = wave % (BN / WN);
  const int64_t kchunks = K / 256;
  int tm, tn;
  tile_of((M + BM - 1) / BM, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t rowbytes = K / 2, srow = K / 16;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  const uint8_t* src[ROUNDS];
  bool code_src[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < C::B_CODES) {
      const int row = p >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = A + (int64_t)min(m0 + row, M - 1) * rowbytes + chunk * 16;
      code_src[r] = true;
    } else if (p < C::A_SC) {
      const int row = (p - C::B_CODES) >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + (int64_t)min(n0 + row, N - 1) * rowbytes + chunk * 16;
      code_src[r] = true;
    } else if (p < C::B_SC) {
      const int q = p - C::A_SC;
      if constexpr (C::MX)
        src[r] = As + (int64_t)min((m0 >> 5) + (q >> 8), (M - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = As + (int64_t)min(m0 + (q >> 4), M - 1) * srow;
      code_src[r] = false;
    } else if (p < C::USED) {
      const int q = p - C::B_SC;
      if constexpr (C::MX)
        src[r] = Bs + (int64_t)min((n0 >> 5) + (q >> 8), (N - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = Bs + (int64_t)min(n0 + (q >> 4), N - 1) * srow;
      code_src[r] = false;
    } else {
      src[r] = As;
      code_src[r] = false;
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
      dma16(src[r] + (code_src[r] ? ks * 64 : (ks >> 1) * C::SC_ADV), slot + r * C::RB + wave * 1024);
  };
  auto dma_tail = [&](int kt) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
    uint8_t* slot = slot_of(kt);
#pragma unroll
    for (int r = H; r < ROUNDS; ++r)
      dma16(src[r] + (code_src[r] ? ks * 64 : (ks >> 1) * C::SC_ADV), slot + r * C::RB + wave * 1024);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  using Frags = NvFrags<TM, TN>;
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
  auto mfmas = [&](const Frags& f) __attribute__((always_inline)) {
    if constexpr (C::MX) {
      // MXINT4: q * 2^e exact in bf16, bf16 MFMA
      float pa[TM], pb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) pa[i] = e8m0_value(f.sa[i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) pb[j] = e8m0_value(f.sb[j]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 av[TM], bv[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = expand8_i4_bf16(f.a[i][t], pa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = expand8_i4_bf16(f.b[j][t], pb[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_bf16(av[i], bv[j], acc[i][j]);
      }
      return;
    }
    _Float16 sa[TM][2], sbv[TN][2];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      sa[i][0] = (_Float16)e4m3_value(f.sa[i] & 0xFFu);
      sa[i][1] = (_Float16)e4m3_value((f.sa[i] >> 8) & 0xFFu);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      sbv[j][0] = (_Float16)e4m3_value(f.sb[j] & 0xFFu);
      sbv[j][1] = (_Float16)e4m3_value((f.sb[j] >> 8) & 0xFFu);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        av[i] = FMT == FP4_FMT_NVINT4 ? expand8_i4_f16(f.a[i][t], sa[i][t >> 1]) : expand8(f.a[i][t], sa[i][t >> 1]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = FMT == FP4_FMT_NVINT4 ? expand8_i4_f16(f.b[j][t], sbv[j][t >> 1]) : expand8(f.b[j][t], sbv[j][t >> 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_f16(av[i], bv[j], acc[i][j]);
    }
  };

  if (kt0 < kt1) {
    // Same schedule as the MXFP4 kernel: step 1's reads and the tail of
    // stage kt+NS-1's DMA with step 0's MFMAs; wait for stage kt+1 and sync;
    // the head of stage kt+NS's DMA and stage kt+1's step-0 reads with step
    // 1's MFMAs.
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
// W4A16 control of the FP4 weight formats; decode streams the weights).  The
// weights' codes and scales go through the same DMA ring as above; each wave
// expands its own B fragments to bf16 in registers (MXFP4: the hardware
// decode applies the E8M0 scale exactly; NVFP4: e2m1 * e4m3 in fp32, exact in
// bf16).  Row tiles are 32 activations high (M is small in decode); the 32
// rows' bf16 activations come straight from global memory into registers,
// one stage ahead.  B's K order within a 64-K step is the FP4 kernels' (lane
// half h, dword t of its 32 codes); A's lane reads the same K positions.
template <int FMT, int BN, int NS>
struct W4Cfg {
  static constexpr int WN = BN / 4, TN = WN / 32;
  static constexpr int SC_BYTES = fmt_mx(FMT) ? (BN / 32) * 256 : BN * 16;
  static constexpr int USED = BN * 64 + SC_BYTES;
  static constexpr int RB = 4096;  // four waves, 1 KB each per round
  static constexpr int ROUNDS = (USED + RB - 1) / RB;
  static constexpr int STAGE = ROUNDS * RB;
  static constexpr int LDS = NS * STAGE;
  static constexpr int A_LOADS = 8;  // 16-byte activation loads per lane per stage
  // vector-memory operations a wave may leave pending once stage kt + 1 has
  // landed: the later stages' DMA (NS - 2 stages) and the next stage's
  // activation loads (the activations run only one stage ahead)
  static constexpr int IN_FLIGHT = (NS - 2) * ROUNDS + A_LOADS;
  static_assert(NS >= 3 && IN_FLIGHT <= 63, "vmcnt range");
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

template <int FMT, int BN, int NS, int YDT, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_w4a16_kernel(
    const uint8_t* __restrict__ A, int64_t lda_bytes, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ bgs, void* __restrict__ Y,
    int64_t ldy, int M, int N, int K, int kchunks, int tiles_n, int kt_per_split,
    float* __restrict__ part) {
  using C = W4Cfg<FMT, BN, NS>;
  constexpr int TN = C::TN, WN = C::WN, ROUNDS = C::ROUNDS;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  tile_of((M + 31) / 32, tiles_n, tm, tn);
  const int m0 = tm * 32, n0 = tn * BN;
  const int64_t rowbytes = K / 2;
  const int KT_total = K / 128;
  const int kt0 = PARTIAL ? blockIdx.y * kt_per_split : 0;
  const int kt1 = PARTIAL ? min(KT_total, kt0 + kt_per_split) : KT_total;

  // DMA sources: B code rows, then the scale pieces of the stage.
  const uint8_t* src[ROUNDS];
  int kind[ROUNDS];  // 0 codes, 1 MX scale tile, 2 NV scale chunk
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * C::RB + tid * 16;
    if (p < BN * 64) {
      const int row = p >> 6, chunk = ((p >> 4) & 3) ^ swz4(row);
      src[r] = B + (int64_t)min(n0 + row, N - 1) * rowbytes + chunk * 16;
      kind[r] = 0;
    } else if (p < C::USED) {
      const int q = p - BN * 64;
      if constexpr (fmt_mx(FMT))
        src[r] = Bs + (int64_t)min((n0 >> 5) + (q >> 8), (N - 1) >> 5) * kchunks * 256 + (q & 255);
      else
        src[r] = Bs + (int64_t)min(n0 + (q >> 4), N - 1) * (K / 16);
      kind[r] = fmt_mx(FMT) ? 1 : 2;
    } else {
      src[r] = Bs;
      kind[r] = 2;
    }
  }
  auto slot_of = [&](int kt) __attribute__((always_inline)) {
    return dyn_lds + (kt % NS) * C::STAGE;
  };
  constexpr int H = ROUNDS / 2;
  auto dma_part = [&](int kt, int r) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
    const int64_t adv = kind[r] == 0 ? ks * 64 : (kind[r] == 1 ? (ks >> 1) * 256 : (ks >> 1) * 16);
    dma16(src[r] + adv, slot_of(kt) + r * C::RB + wave * 1024);
  };

  // activations: lane row m0 + lane % 32 (clamped), K half h = lane / 32
  const uint8_t* arow = A + (int64_t)min(m0 + (lane & 31), M - 1) * lda_bytes + (lane >> 5) * 64;
  u32x4 a_cur[8], a_nxt[8];
  auto load_a = [&](int kt, u32x4* dst) __attribute__((always_inline)) {
    const int ks = min(kt, kt1 - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dst[s * 4 + t] = *reinterpret_cast<const u32x4*>(arow + (int64_t)ks * 256 + s * 128 + t * 16);
  };

  f32x16 acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

  // one 64-K step: B fragments of the step from LDS, expanded per MFMA
  auto step = [&](int kt, int s, const u32x4* a) __attribute__((always_inline)) {
    const uint8_t* slot = slot_of(kt);
    const int q = s * 2 + (lane >> 5);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wave * WN + j * 32 + (lane & 31);
      const u32x4 codes = *reinterpret_cast<const u32x4*>(slot + row * 64 + ((q ^ swz4(row)) * 16));
      if constexpr (fmt_mx(FMT)) {
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(slot + BN * 64 + (row >> 5) * 256 + (lane & 31) * 4 +
                                                                (lane >> 5) * 128);
        const uint32_t code = (sc >> (8 * (2 * (kt & 1) + s))) & 0xFFu;
        if constexpr (fmt_int(FMT)) {
          const float p = e8m0_value(code);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[j] = mfma_bf16(a[s * 4 + t], expand8_i4_bf16(codes[t], p), acc[j]);
        } else {
          const float scale = e8m0_as_cvt_scale(code);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[j] = mfma_bf16(a[s * 4 + t], expand8_bf16_mx(codes[t], scale), acc[j]);
        }
      } else {
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(
            slot + BN * 64 + row * 16 + 8 * (kt & 1) + 4 * s + 2 * (lane >> 5));
        const float s0 = e4m3_value(sc2 & 0xFFu), s1 = e4m3_value(sc2 >> 8);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[j] = mfma_bf16(a[s * 4 + t],
                             fmt_int(FMT) ? expand8_i4_bf16(codes[t], t < 2 ? s0 : s1)
                                          : expand8_bf16_nv(codes[t], t < 2 ? s0 : s1),
                             acc[j]);
      }
    }
  };

  if (kt0 < kt1) {
    load_a(kt0, a_cur);
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r) dma_part(kt0 + i, r);
#pragma unroll
    for (int r = 0; r < H; ++r) dma_part(kt0 + NS - 1, r);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * ROUNDS + H, 15));
    __builtin_amdgcn_s_barrier();
    for (int kt = kt0; kt < kt1; ++kt) {
      // first half: next stage's activations, the tail of stage kt+NS-1's
      // DMA, step 0; then wait for stage kt+1 and sync; second half: the
      // head of stage kt+NS's DMA (into slot kt, read by nobody after the
      // sync of the next iteration) and step 1.
      load_a(kt + 1, a_nxt);
#pragma unroll
      for (int r = H; r < ROUNDS; ++r) dma_part(kt + NS - 1, r);
      step(kt, 0, a_cur);
      step(kt, 1, a_cur);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::IN_FLIGHT, 0));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < H; ++r) dma_part(kt + NS, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) a_cur[i] = a_nxt[i];
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  }

  const float g = (!fmt_mx(FMT) && !PARTIAL) ? *bgs : 1.0f;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = m0 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
      const int col = n0 + wave * WN + j * 32 + (lane & 31);
      if (row < M && col < N) {
        if constexpr (PARTIAL)
          part[((int64_t)blockIdx.y * M + row) * N + col] = acc[j][e];
        else
          store_out<YDT>(Y, ldy, row, col, acc[j][e] * g);
      }
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
                         const uint8_t* b, const uint8_t* bs, void* y, int ydt, int64_t ldy,
                         int splits, int kt_per, float* part, hipStream_t st) {
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  const int kchunks = (int)mx_gemm_kchunks(K);
  const size_t lds = MxCfg<BM, BN, WM, WN, NS>::LDS;
  hipError_t e;
  if (splits > 1) {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_F32, true><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  } else if (ydt == FP4_DT_F32) {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_F32, false><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  } else {
    if ((e = mx_lds_attr<BM, BN, WM, WN, NS, FP4_DT_BF16, false>()) != hipSuccess) return e;
    gemm_mx_kernel<BM, BN, WM, WN, NS, FP4_DT_BF16, false><<<grid, (MxCfg<BM, BN, WM, WN, NS>::NW * 64), lds, st>>>(
        a, as, b, bs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  }
  return hipGetLastError();
}

template <int FMT, int BM, int BN, int WM, int WN, int NS, int YDT, bool PARTIAL>
hipError_t nv_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, NvCfg<BM, BN, WM, WN, NS, FMT>::LDS);
  return status;
}

template <int BM, int BN, int WM, int WN, int NS, int FMT = FP4_FMT_NVFP4>
hipError_t launch_nv_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                         const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                         void* y, int ydt, int64_t ldy, int splits, int kt_per, float* part,
                         hipStream_t st) {
  using C = NvCfg<BM, BN, WM, WN, NS, FMT>;
  const int tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(((M + BM - 1) / BM) * tiles_n), (unsigned)splits);
  hipError_t e;
  if (splits > 1) {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, true><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part);
  } else if (ydt == FP4_DT_F32) {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_F32, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part);
  } else {
    if ((e = nv_lds_attr<FMT, BM, BN, WM, WN, NS, FP4_DT_BF16, false>()) != hipSuccess) return e;
    gemm_nv_ring_kernel<FMT, BM, BN, WM, WN, NS, FP4_DT_BF16, false><<<grid, C::NW * 64, C::LDS, st>>>(
        a, as, ags, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, tiles_n, kt_per, part);
  }
  return hipGetLastError();
}

template <int FMT, int YDT, bool PARTIAL>
hipError_t w4_lds_attr() {
  static hipError_t status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemm_w4a16_kernel<FMT, 256, 3, YDT, PARTIAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, W4Cfg<FMT, 256, 3>::LDS);
  return status;
}

template <int FMT>
hipError_t launch_w4_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda_bytes,
                         const uint8_t* b, const uint8_t* bs, const float* bgs, void* y, int ydt,
                         int64_t ldy, int splits, int kt_per, float* part, hipStream_t st) {
  using C = W4Cfg<FMT, 256, 3>;
  const int tiles_n = (int)((N + 255) / 256);
  const dim3 grid((unsigned)(((M + 31) / 32) * tiles_n), (unsigned)splits);
  const int kchunks = (int)mx_gemm_kchunks(K);
  hipError_t e;
  if (splits > 1) {
    if ((e = w4_lds_attr<FMT, FP4_DT_F32, true>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, 256, 3, FP4_DT_F32, true><<<grid, 256, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  } else if (ydt == FP4_DT_F32) {
    if ((e = w4_lds_attr<FMT, FP4_DT_F32, false>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, 256, 3, FP4_DT_F32, false><<<grid, 256, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  } else {
    if ((e = w4_lds_attr<FMT, FP4_DT_BF16, false>()) != hipSuccess) return e;
    gemm_w4a16_kernel<FMT, 256, 3, FP4_DT_BF16, false><<<grid, 256, C::LDS, st>>>(
        a, lda_bytes, b, bs, bgs, y, ldy, (int)M, (int)N, (int)K, kchunks, tiles_n, kt_per, part);
  }
  return hipGetLastError();
}

// Split factor of the weight-only GEMM: 32-row tiles, split K while fewer than
// 512 workgroups would run (at least 4 stages per slice, slices of whole
// 256-K scale chunks).
struct W4Plan {
  int splits, kt_per;
};
W4Plan plan_w4(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 31) / 32) * ((N + 255) / 256);
  const int KT = (int)(K / 128);
  int splits = 1;
  while (tiles * splits * 2 <= 512 && splits < 16 && KT / (splits * 2) >= 4) splits *= 2;
  int kt_per = (KT + splits - 1) / splits;
  kt_per += kt_per & 1;
  return W4Plan{splits, kt_per};
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
template <int YDT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 int splits, int M, int N,
                                                                 void* __restrict__ Y,
                                                                 int64_t ldy,
                                                                 const float* __restrict__ ga,
                                                                 const float* __restrict__ gb) {
  const int64_t total = (int64_t)M * N;
  const bool scaled = ga != nullptr || gb != nullptr;
  const float g = (ga ? *ga : 1.0f) * (gb ? *gb : 1.0f);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * total + i];
    const int row = (int)(i / N), col = (int)(i - (int64_t)row * N);
    store_out<YDT>(Y, ldy, row, col, scaled ? s * g : s);
  }
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, void* y,
                                int ydt, int64_t ldy, const float* ga, const float* gb,
                                hipStream_t st) {
  int64_t g = (M * N + kThreads - 1) / kThreads;
  if (g > 8192) g = 8192;
  if (ydt == FP4_DT_F32)
    splitk_reduce_kernel<FP4_DT_F32><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
  else
    splitk_reduce_kernel<FP4_DT_BF16><<<(int)g, kThreads, 0, st>>>(part, splits, (int)M, (int)N, y, ldy, ga, gb);
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
    while (tiles * splits * 2 <= cap && splits < 16 && KT / (splits * 2) >= 4) splits *= 2;
  p.splits = splits;
  p.kt_per = (KT + splits - 1) / splits;
  p.kt_per += p.kt_per & 1;
  return p;
}

}  // namespace

namespace fp4lib {

size_t gemm_mx_workspace(int64_t M, int64_t N, int64_t K) {
  MxPlan p = plan_mx(M, N, K, 128, true);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_mx(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const uint8_t* b, const uint8_t* bs, void* y, int ydt, int64_t ldy,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {  // empty sum
    zero_out_kernel<<<256, kThreads, 0, st>>>(y, ydt, (int)M, (int)N, ldy);
    return hipGetLastError();
  }
  MxPlan p = plan_mx(M, N, K, 128, true);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_mx_workspace(M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  if (p.cfg == 0)
    e = launch_mx_cfg<256, 256, 128, 64, 4>(M, N, K, a, as, b, bs, y, ydt, ldy, splits, kt_per, part, st);
  else if (p.cfg == 1)
    e = launch_mx_cfg<128, 128, 64, 64, 4>(M, N, K, a, as, b, bs, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_mx_cfg<32, 128, 32, 32, 6>(M, N, K, a, as, b, bs, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, nullptr, nullptr, st);
}

size_t gemm_nv_workspace(int64_t M, int64_t N, int64_t K) {
  if (K % 256 != 0 || K == 0) return 0;
  MxPlan p = plan_mx(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// The ring GEMM with expanded operands for INT4 elements: NVINT4 on fp16
// MFMA (n * e4m3 exact in fp16), MXINT4 on bf16 MFMA (n * 2^e exact in bf16).
template <int FMT>
hipError_t launch_ring_int4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                            const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                            void* y, int ydt, int64_t ldy, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  MxPlan p = plan_mx(M, N, K);
  const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_nv_workspace(M, N, K);
  const int splits = split ? p.splits : 1;
  const int kt_per = split ? p.kt_per : (int)(K / 128);
  float* part = static_cast<float*>(ws);
  hipError_t e;
  if (p.cfg == 0)
    e = launch_nv_cfg<256, 256, 128, 128, 3, FMT>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  else if (p.cfg == 1)
    e = launch_nv_cfg<128, 128, 64, 64, 3, FMT>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_nv_cfg<32, 256, 32, 64, 3, FMT>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, fmt_mx(FMT) ? nullptr : ags,
                              fmt_mx(FMT) ? nullptr : bgs, st);
}

hipError_t launch_gemm_int4(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                            const uint8_t* as, const float* ags, const uint8_t* b, const uint8_t* bs,
                            const float* bgs, void* y, int ydt, int64_t ldy, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    zero_out_kernel<<<256, kThreads, 0, st>>>(y, ydt, (int)M, (int)N, ldy);
    return hipGetLastError();
  }
  if (fmt == FP4_FMT_MXINT4)
    return launch_ring_int4<FP4_FMT_MXINT4>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, ws, ws_bytes, st);
  return launch_ring_int4<FP4_FMT_NVINT4>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, ws, ws_bytes, st);
}

hipError_t launch_gemm_nv(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                          const float* ags, const uint8_t* b, const uint8_t* bs, const float* bgs,
                          void* y, int ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K % 256 == 0 && K > 0) {
    // LDS ring with in-register fp16 expansion; tiles and split-K as for MXFP4
    MxPlan p = plan_mx(M, N, K);
    const bool split = p.splits > 1 && ws != nullptr && ws_bytes >= gemm_nv_workspace(M, N, K);
    const int splits = split ? p.splits : 1;
    const int kt_per = split ? p.kt_per : (int)(K / 128);
    float* part = static_cast<float*>(ws);
    hipError_t e;
    if (p.cfg == 0)
      e = launch_nv_cfg<256, 256, 128, 128, 3>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
    else if (p.cfg == 1)
      e = launch_nv_cfg<128, 128, 64, 64, 3>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
    else
      e = launch_nv_cfg<32, 256, 32, 64, 3>(M, N, K, a, as, ags, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
    if (e != hipSuccess || !split) return e;
    return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy, ags, bgs, st);
  }
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

size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K) {
  if (K % 256 != 0 || K == 0 || M == 0 || N == 0) return 0;
  W4Plan p = plan_w4(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_w4a16(int fmt, int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                             const uint8_t* b, const uint8_t* bs, const float* bgs, void* y, int ydt,
                             int64_t ldy, void* ws, size_t ws_bytes, hipStream_t st) {
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
    e = launch_w4_fmt<FP4_FMT_MXFP4>(M, N, K, ab, lda * 2, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  else if (fmt == FP4_FMT_NVFP4)
    e = launch_w4_fmt<FP4_FMT_NVFP4>(M, N, K, ab, lda * 2, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  else if (fmt == FP4_FMT_MXINT4)
    e = launch_w4_fmt<FP4_FMT_MXINT4>(M, N, K, ab, lda * 2, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  else
    e = launch_w4_fmt<FP4_FMT_NVINT4>(M, N, K, ab, lda * 2, b, bs, bgs, y, ydt, ldy, splits, kt_per, part, st);
  if (e != hipSuccess || !split) return e;
  return launch_splitk_reduce(part, splits, M, N, y, ydt, ldy,
                              fmt_mx(fmt) ? nullptr : bgs, nullptr, st);
}

}  // namespace fp4lib
