// MFMA main loop shared by every contraction of the encode path.
//
// One workgroup computes a BM x BN tile of C = A * B^T where every row of A
// and of B is K-contiguous in HBM (the "NT" form: token rows of kv, packed
// weight rows, reference rows all have their contraction index innermost).
// Its waves form a WGM x WGN grid (2 x 2 by default; the bf16 loop also runs
// 2 x 4); wave (wm, wn) owns the (BM/WGM) x (BN/WGN) sub-tile as fragments of
// 32 x 32 fp32 accumulators.
//
//  - bf16 operands use v_mfma_f32_32x32x16_bf16 (products exact, fp32 sums);
//    fp32 operands use v_mfma_f32_32x32x2_f32.  Both write the same 32 x 32
//    accumulator layout, so every epilogue serves both element types.
//  - bf16: an LDS-DMA ring (gemm_mainloop_dma below): the operands go from
//    HBM/L2 straight into NS stages of LDS, no register staging.
//  - fp32 (gemm_mainloop, next): K advances 128 bytes (32 values) per stage;
//    stages are double-buffered in LDS and each thread stages 16-byte chunks
//    through registers, so the next stage's global loads are in flight
//    while the current stage feeds the matrix cores.  One barrier per
//    stage.  LDS rows are padded by 16 bytes: the 32 lanes of a half-wave
//    that read 32 consecutive rows at the same K offset hit distinct banks.
//
// tile_product (at the end) is the entry: callers give the first byte of
// each tile row (rows past the end of a matrix clamped to a valid row,
// their results masked by the epilogue).
#pragma once
#include <type_traits>

#include "rkv_device.h"

namespace rkv {

template <typename E, int BM, int BN>
struct Tile {
  static constexpr int kThreads = 256;
  static constexpr int kStage = 128;             // K bytes per stage
  static constexpr int kRow = kStage + 16;       // padded LDS row, bytes
  static constexpr int kWM = BM / 2, kWN = BN / 2;
  static constexpr int kTM = kWM / 32, kTN = kWN / 32;
  static constexpr int kLdA = BM / 32, kLdB = BN / 32;
  static constexpr int kLds = 2 * (BM + BN) * kRow;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must hold 2x2 waves of 32x32 fragments");
};

template <typename E>
struct Mfma;

template <>
struct Mfma<uint16_t> {  // bf16 bits
  static constexpr int kSteps = 4;  // 16 elements (32 bytes) of K per MFMA
  typedef bf16x8 Frag;
  __device__ __forceinline__ static Frag load(const char* row, int step, int lane) {
    return *reinterpret_cast<const bf16x8*>(row + step * 32 + (lane >> 5) * 16);
  }
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int kSteps = 16;  // 2 elements (8 bytes) of K per MFMA
  typedef float Frag;
  __device__ __forceinline__ static Frag load(const char* row, int step, int lane) {
    return *reinterpret_cast<const float*>(row + step * 8 + (lane >> 5) * 4);
  }
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename E, int BM, int BN>
__device__ __forceinline__ void gemm_mainloop(const char* (&pa)[BM / 32],
                                              const char* (&pb)[BN / 32], int stages,
                                              char* lds,
                                              f32x16 (&acc)[BM / 64][BN / 64]) {
  using TL = Tile<E, BM, BN>;
  using M = Mfma<E>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  char* sA0 = lds;
  char* sB0 = lds + BM * TL::kRow;
  constexpr int kBuf = (BM + BN) * TL::kRow;
  const int srow = tid >> 3, scol = (tid & 7) * 16;

#pragma unroll
  for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
    for (int j = 0; j < TL::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 ra[TL::kLdA], rb[TL::kLdB];
#pragma unroll
  for (int i = 0; i < TL::kLdA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i]);
#pragma unroll
  for (int i = 0; i < TL::kLdB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i]);
#pragma unroll
  for (int i = 0; i < TL::kLdA; ++i)
    *reinterpret_cast<u32x4*>(sA0 + (srow + 32 * i) * TL::kRow + scol) = ra[i];
#pragma unroll
  for (int i = 0; i < TL::kLdB; ++i)
    *reinterpret_cast<u32x4*>(sB0 + (srow + 32 * i) * TL::kRow + scol) = rb[i];
  __syncthreads();

  const int arow = wm * TL::kWM + (lane & 31);
  const int brow = wn * TL::kWN + (lane & 31);
  for (int kt = 0; kt < stages; ++kt) {
    const int cur = (kt & 1) * kBuf;
    const bool more = kt + 1 < stages;
    if (more) {
      const int off = (kt + 1) * TL::kStage;
#pragma unroll
      for (int i = 0; i < TL::kLdA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + off);
#pragma unroll
      for (int i = 0; i < TL::kLdB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + off);
    }
    const char* sA = sA0 + cur;
    const char* sB = sB0 + cur;
#pragma unroll
    for (int st = 0; st < M::kSteps; ++st) {
      typename M::Frag fa[TL::kTM], fb[TL::kTN];
#pragma unroll
      for (int i = 0; i < TL::kTM; ++i) fa[i] = M::load(sA + (arow + 32 * i) * TL::kRow, st, lane);
#pragma unroll
      for (int j = 0; j < TL::kTN; ++j) fb[j] = M::load(sB + (brow + 32 * j) * TL::kRow, st, lane);
#pragma unroll
      for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
        for (int j = 0; j < TL::kTN; ++j) acc[i][j] = M::mma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      const int nxt = kBuf - cur;
#pragma unroll
      for (int i = 0; i < TL::kLdA; ++i)
        *reinterpret_cast<u32x4*>(sA0 + nxt + (srow + 32 * i) * TL::kRow + scol) = ra[i];
#pragma unroll
      for (int i = 0; i < TL::kLdB; ++i)
        *reinterpret_cast<u32x4*>(sB0 + nxt + (srow + 32 * i) * TL::kRow + scol) = rb[i];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 main loop: LDS-DMA ring (gfx950 buffer_load_dwordx4 ... lds, or
// global_load_lds_dwordx4 where a tile spans more than a buffer reaches).
//
// Same tile and accumulator layout as gemm_mainloop, but:
//  - operands travel HBM/L2 -> LDS directly (no VGPR staging), NS stages of
//    SB bytes of K per row in flight, so a stage is requested NS-1 stages
//    before it is consumed;
//  - LDS rows are SB bytes, unpadded; the 16-byte slot of each row is XOR-
//    swizzled (swz) so the rows a half-wave reads at one K offset spread
//    over the banks (the DMA writes 1 KB contiguous per wave instruction,
//    so the swizzle is applied on the global side: lane l of a DMA
//    instruction fetches slot (l % kSlots) ^ swz(row));
//  - fragments are double-buffered: the next k-step's reads are issued
//    between this k-step's MFMAs (sched_group_barrier keeps that order);
//  - waits are explicit s_waitcnt vmcnt(n) + a bare s_barrier (no fence), so
//    younger stages stay in flight across the barrier.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int BM, int BN, int SB, int NS, int WGM = 2, int WGN = 2>
struct DmaTile {
  static constexpr int kWaves = WGM * WGN;        // wave grid WGM x WGN
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kSlots = SB / 16;          // 16-byte slots per LDS row
  static constexpr int kRowsPerKB = 1024 / SB;    // rows per DMA wave instruction
  static constexpr int kStage = (BM + BN) * SB;   // bytes per stage
  static constexpr int kLds = NS * kStage;
  static constexpr int kWM = BM / WGM, kWN = BN / WGN, kTM = kWM / 32, kTN = kWN / 32;
  static constexpr int kSteps = SB / 32;          // 32x32x16 k-steps per stage
  // DMA instructions per wave per stage
  static constexpr int kLdA = BM * SB / (1024 * kWaves), kLdB = BN * SB / (1024 * kWaves);
  static constexpr int kLd = kLdA + kLdB;
  static_assert(kSteps % 2 == 0, "fragment double-buffering pairs k-steps");
  static_assert(NS >= 2, "a stage is requested at least one stage ahead");
  static_assert(kLdA >= 1 && kLdB >= 1, "each wave feeds part of A and of B");
  static_assert(BM * SB == kLdA * 1024 * kWaves && BN * SB == kLdB * 1024 * kWaves,
                "the DMA instructions of a stage cover every row of A and of B");
  static_assert(kLd * (NS - 2 > 0 ? NS - 2 : 0) <= 31, "vmcnt window");
};

// (chosen by measurement: SQ_LDS_BANK_CONFLICT reads zero for the fragment
// reads of both row widths with these two maps)
template <int SB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (SB == 64) return (r >> 2) & 3;
  else return (r ^ (r >> 3)) & 7;
}

// Tile-local row fed by DMA instruction i of this lane, and the byte offset
// of the (swizzled) K slot it fetches within a stage.
template <typename TL, int SB>
__device__ __forceinline__ int dma_row(int i, int per_wave) {
  return ((threadIdx.x >> 6) * per_wave + i) * TL::kRowsPerKB + (threadIdx.x & 63) / TL::kSlots;
}
template <typename TL, int SB>
__device__ __forceinline__ int dma_slot(int row) {
  return (((threadIdx.x & 63) % TL::kSlots) ^ swz<SB>(row)) << 4;
}

// s_waitcnt vmcnt(n) lgkmcnt(0)
__device__ __forceinline__ void wait_vm_lgkm(int n) {
#define RKV_WVM(N) \
  case N: __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4)); break;
  switch (n) {
    RKV_WVM(0) RKV_WVM(1) RKV_WVM(2) RKV_WVM(3) RKV_WVM(4) RKV_WVM(5) RKV_WVM(6) RKV_WVM(7)
    RKV_WVM(8) RKV_WVM(9) RKV_WVM(10) RKV_WVM(11) RKV_WVM(12) RKV_WVM(13) RKV_WVM(14)
    RKV_WVM(15) RKV_WVM(16) RKV_WVM(17) RKV_WVM(18) RKV_WVM(19) RKV_WVM(20) RKV_WVM(21)
    RKV_WVM(22) RKV_WVM(23) RKV_WVM(24) RKV_WVM(25) RKV_WVM(26) RKV_WVM(27) RKV_WVM(28)
    RKV_WVM(29) RKV_WVM(30) RKV_WVM(31)
    default: __builtin_amdgcn_s_waitcnt(0x7 << 4); break;  // vmcnt(0) lgkmcnt(0)
  }
#undef RKV_WVM
}

// Workgroup barrier without a memory fence (the waits above order memory);
// the empty asm statements stop the compiler moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Where DMA instruction i of this lane reads at K stage 0 (row base +
// dma_slot; rows past the end must point at a valid row), in one of two
// forms chosen by BUF:
//  - global form (global_load_lds): pa[i] / pb[i], a 64-bit lane address;
//  - buffer form (buffer_load ... lds): va[i] / vb[i], a 32-bit byte offset
//    in the buffer resource ra / rb, with the stage offset in an SGPR, so a
//    stage costs no vector address arithmetic (measured 4-5% faster on the
//    token-projection shape).
template <int BM, int BN, int SB, int NS, int WGM, int WGN, bool BUF>
__device__ __forceinline__ void gemm_mainloop_dma(const char* const* pa, const char* const* pb,
                                                  const uint32_t* va, const uint32_t* vb,
                                                  __amdgpu_buffer_rsrc_t ra,
                                                  __amdgpu_buffer_rsrc_t rb, int KT, char* lds,
                                                  f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  using TL = DmaTile<BM, BN, SB, NS, WGM, WGN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
    for (int j = 0; j < TL::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto issue = [&](int s) {
    char* buf = lds + (s % NS) * TL::kStage;
#pragma unroll
    for (int i = 0; i < TL::kLdA; ++i) {
      lds_ptr_t dst = (lds_ptr_t)(buf + (wave * TL::kLdA + i) * 1024);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, va[i], s * SB, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(pa[i] + size_t(s) * SB, dst, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TL::kLdB; ++i) {
      lds_ptr_t dst = (lds_ptr_t)(buf + BM * SB + (wave * TL::kLdB + i) * 1024);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, vb[i], s * SB, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(pb[i] + size_t(s) * SB, dst, 16, 0, 0);
    }
  };
  int offA[TL::kTM], swA[TL::kTM], offB[TL::kTN], swB[TL::kTN];
#pragma unroll
  for (int i = 0; i < TL::kTM; ++i) {
    const int r = wm * TL::kWM + i * 32 + (lane & 31);
    offA[i] = r * SB;
    swA[i] = swz<SB>(r);
  }
#pragma unroll
  for (int j = 0; j < TL::kTN; ++j) {
    const int r = wn * TL::kWN + j * 32 + (lane & 31);
    offB[j] = BM * SB + r * SB;
    swB[j] = swz<SB>(r);
  }
  const int hi = lane >> 5;
  bf16x8 fa[2][TL::kTM], fb[2][TL::kTN];
  auto load_frags = [&](int stage, int st, int p) {
    const char* buf = lds + (stage % NS) * TL::kStage;
    const int kc = 2 * st + hi;
#pragma unroll
    for (int i = 0; i < TL::kTM; ++i)
      fa[p][i] = *reinterpret_cast<const bf16x8*>(buf + offA[i] + ((kc ^ swA[i]) << 4));
#pragma unroll
    for (int j = 0; j < TL::kTN; ++j)
      fb[p][j] = *reinterpret_cast<const bf16x8*>(buf + offB[j] + ((kc ^ swB[j]) << 4));
  };

  // One stage: its MFMAs, with the next k-step's fragment reads between
  // them.  ISSUE: the stage NS-1 ahead is requested first; NEXT: a later
  // stage exists, so the last k-step waits for it, syncs and reads its first
  // fragments before its own MFMAs (whose fragments are already in
  // registers).  Both are compile-time, so no branch makes the compiler
  // drain those reads before the MFMAs.
  auto stage = [&](int kt, auto issue_c, auto next_c, int younger) {
    constexpr bool kIssue = decltype(issue_c)::value, kNext = decltype(next_c)::value;
    if constexpr (kIssue) issue(kt + NS - 1);
#pragma unroll
    for (int st = 0; st < TL::kSteps; ++st) {
      const int p = st & 1;
      if (st + 1 < TL::kSteps) {
        load_frags(kt, st + 1, p ^ 1);
      } else if constexpr (kNext) {
        // stage kt+1 must have landed (`younger` later stages may stay in
        // flight), and every wave must be done with the buffer the next
        // issue reuses
        wait_vm_lgkm(TL::kLd * younger);
        block_barrier();
        load_frags(kt + 1, 0, p ^ 1);
      }
#pragma unroll
      for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
        for (int j = 0; j < TL::kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[p][i], fb[p][j], acc[i][j], 0, 0, 0);
      constexpr int kMfma = TL::kTM * TL::kTN, kReads = TL::kTM + TL::kTN;
#pragma unroll
      for (int x = 0; x < kReads; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using yes = std::true_type;
  using no = std::false_type;

  const int pre = NS - 1 < KT ? NS - 1 : KT;
  for (int s = 0; s < pre; ++s) issue(s);
  wait_vm_lgkm(TL::kLd * (pre - 1));
  block_barrier();
  load_frags(0, 0, 0);
  int kt = 0;
  // stages that request a later one (then NS-2 younger stages stay in flight)
  for (; kt + NS - 1 < KT; ++kt) stage(kt, yes{}, yes{}, NS - 2);
  // the last NS-2 stages but one: nothing left to request
  for (; kt + 1 < KT; ++kt) stage(kt, no{}, yes{}, KT - 2 - kt);
  if (kt < KT) stage(kt, no{}, no{}, 0);
  // leave no LDS read in flight: callers reuse the LDS right away
  __builtin_amdgcn_s_waitcnt((0xF | (3 << 14)) | (0x7 << 4));
  block_barrier();
}

// ---------------------------------------------------------------------------
// bf16 main loop for an A operand carried as (hi, lo) bf16 pairs, x = hi +
// lo to about 16 significant bits.  An A row holds, for every 8 consecutive
// K features, 16 bytes of hi values followed by 16 bytes of lo values; a B
// row holds each feature once.  One B fragment then feeds two MFMAs, hi * b
// and lo * b, into the same accumulator, so B moves half the bytes that a
// B row with every value duplicated would, and is read from LDS half as
// often.
//  - a stage carries SB bytes of every A row (SB/4 features) and SB/2 bytes
//    of every B row, both through the LDS-DMA ring as in gemm_mainloop_dma;
//  - a k-step covers 16 features: lane half h reads the A slots 4st + 2h
//    (hi) and 4st + 2h + 1 (lo) and the B slot 2st + h;
//  - each k-step runs as two phases, hi then lo, whose A fragments alternate
//    between two register buffers (the next phase's reads are issued between
//    this phase's MFMAs); B fragments are double-buffered across k-steps.
//    The hi and lo MFMAs of one accumulator lie kTM*kTN MFMAs apart.
template <int BM, int BN, int SB, int NS, int WGM = 2, int WGN = 2>
struct DmaTileHL {
  static constexpr int SBB = SB / 2;              // B bytes per row per stage
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kSlotsA = SB / 16, kSlotsB = SBB / 16;
  static constexpr int kRowsPerKBA = 1024 / SB, kRowsPerKBB = 1024 / SBB;
  static constexpr int kStageA = BM * SB;
  static constexpr int kStage = BM * SB + BN * SBB;
  static constexpr int kLds = NS * kStage;
  static constexpr int kWM = BM / WGM, kWN = BN / WGN, kTM = kWM / 32, kTN = kWN / 32;
  static constexpr int kSteps = SB / 64;          // 16-feature k-steps per stage
  static constexpr int kLdA = BM * SB / (1024 * kWaves), kLdB = BN * SBB / (1024 * kWaves);
  static constexpr int kLd = kLdA + kLdB;
  static_assert(SB == 128, "A stages of 128 bytes, B of 64 (the swizzles measured conflict-free)");
  static_assert(NS >= 2, "a stage is requested at least one stage ahead");
  static_assert(kLdA >= 1 && kLdB >= 1, "each wave feeds part of A and of B");
  static_assert(BM * SB == kLdA * 1024 * kWaves && BN * SBB == kLdB * 1024 * kWaves,
                "the DMA instructions of a stage cover every row of A and of B");
  static_assert(kTM + kTN <= kTM * kTN, "a phase's reads fit between its MFMAs");
  static_assert(kLd * (NS - 2 > 0 ? NS - 2 : 0) <= 31, "vmcnt window");
};

template <int BM, int BN, int SB, int NS, int WGM, int WGN, bool BUF>
__device__ __forceinline__ void gemm_mainloop_dma_hl(const char* const* pa, const char* const* pb,
                                                     const uint32_t* va, const uint32_t* vb,
                                                     __amdgpu_buffer_rsrc_t ra,
                                                     __amdgpu_buffer_rsrc_t rb, int KT, char* lds,
                                                     f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  using TL = DmaTileHL<BM, BN, SB, NS, WGM, WGN>;
  constexpr int SBB = TL::SBB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
    for (int j = 0; j < TL::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto issue = [&](int s) {
    char* buf = lds + (s % NS) * TL::kStage;
#pragma unroll
    for (int i = 0; i < TL::kLdA; ++i) {
      lds_ptr_t dst = (lds_ptr_t)(buf + (wave * TL::kLdA + i) * 1024);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, va[i], s * SB, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(pa[i] + size_t(s) * SB, dst, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < TL::kLdB; ++i) {
      lds_ptr_t dst = (lds_ptr_t)(buf + TL::kStageA + (wave * TL::kLdB + i) * 1024);
      if constexpr (BUF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, vb[i], s * SBB, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(pb[i] + size_t(s) * SBB, dst, 16, 0, 0);
    }
  };
  int offA[TL::kTM], swA[TL::kTM], offB[TL::kTN], swB[TL::kTN];
#pragma unroll
  for (int i = 0; i < TL::kTM; ++i) {
    const int r = wm * TL::kWM + i * 32 + (lane & 31);
    offA[i] = r * SB;
    swA[i] = swz<SB>(r);
  }
#pragma unroll
  for (int j = 0; j < TL::kTN; ++j) {
    const int r = wn * TL::kWN + j * 32 + (lane & 31);
    offB[j] = TL::kStageA + r * SBB;
    swB[j] = swz<SBB>(r);
  }
  const int hi = lane >> 5;
  bf16x8 fa[2][TL::kTM], fb[2][TL::kTN];
  // A fragments of k-step st, hi (part 0) or lo (part 1) values, into fa[part]
  auto load_a = [&](int stage, int st, int part) {
    const char* buf = lds + (stage % NS) * TL::kStage;
    const int kc = 4 * st + 2 * hi + part;
#pragma unroll
    for (int i = 0; i < TL::kTM; ++i)
      fa[part][i] = *reinterpret_cast<const bf16x8*>(buf + offA[i] + ((kc ^ swA[i]) << 4));
  };
  auto load_b = [&](int stage, int st, int p) {
    const char* buf = lds + (stage % NS) * TL::kStage;
    const int kc = 2 * st + hi;
#pragma unroll
    for (int j = 0; j < TL::kTN; ++j)
      fb[p][j] = *reinterpret_cast<const bf16x8*>(buf + offB[j] + ((kc ^ swB[j]) << 4));
  };
  constexpr int kMfma = TL::kTM * TL::kTN;
  auto mfmas = [&](int part, int p) {
#pragma unroll
    for (int i = 0; i < TL::kTM; ++i)
#pragma unroll
      for (int j = 0; j < TL::kTN; ++j)
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[part][i], fb[p][j], acc[i][j], 0, 0, 0);
  };
  // one MFMA, one LDS read, ... then the phase's remaining MFMAs
  auto order = [](auto reads_c) {
    constexpr int kReads = decltype(reads_c)::value;
#pragma unroll
    for (int x = 0; x < kReads; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (kMfma > kReads) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using kReadsHi = std::integral_constant<int, TL::kTM>;
  using kReadsLo = std::integral_constant<int, TL::kTM + TL::kTN>;
  using kReadsNone = std::integral_constant<int, 0>;

  // One stage, as in gemm_mainloop_dma: ISSUE requests the stage NS-1
  // ahead first; NEXT (a later stage exists) makes the last phase wait for
  // it, sync and read its first fragments before its own MFMAs.
  auto stage = [&](int kt, auto issue_c, auto next_c, int younger) {
    constexpr bool kIssue = decltype(issue_c)::value, kNext = decltype(next_c)::value;
    if constexpr (kIssue) issue(kt + NS - 1);
#pragma unroll
    for (int st = 0; st < TL::kSteps; ++st) {
      const int p = st & 1;
      // hi phase: the lo fragments of this k-step are read meanwhile
      load_a(kt, st, 1);
      mfmas(0, p);
      order(kReadsHi{});
      // lo phase: the next k-step's hi and B fragments are read meanwhile
      if (st + 1 < TL::kSteps) {
        load_a(kt, st + 1, 0);
        load_b(kt, st + 1, p ^ 1);
        mfmas(1, p);
        order(kReadsLo{});
      } else if constexpr (kNext) {
        wait_vm_lgkm(TL::kLd * younger);
        block_barrier();
        load_a(kt + 1, 0, 0);
        load_b(kt + 1, 0, p ^ 1);
        mfmas(1, p);
        order(kReadsLo{});
      } else {
        mfmas(1, p);
        order(kReadsNone{});
      }
    }
  };
  static_assert(TL::kSteps % 2 == 0 || TL::kSteps == 1, "B buffers alternate across stages");
  using yes = std::true_type;
  using no = std::false_type;

  const int pre = NS - 1 < KT ? NS - 1 : KT;
  for (int s = 0; s < pre; ++s) issue(s);
  wait_vm_lgkm(TL::kLd * (pre - 1));
  block_barrier();
  load_a(0, 0, 0);
  load_b(0, 0, 0);
  int kt = 0;
  for (; kt + NS - 1 < KT; ++kt) stage(kt, yes{}, yes{}, NS - 2);
  for (; kt + 1 < KT; ++kt) stage(kt, no{}, yes{}, KT - 2 - kt);
  if (kt < KT) stage(kt, no{}, no{}, 0);
  __builtin_amdgcn_s_waitcnt((0xF | (3 << 14)) | (0x7 << 4));
  block_barrier();
}

// One workgroup tile of C = A * B^T with A as (hi, lo) pairs (layout above):
// rowA(r) / rowB(r) return the first byte of tile-local row r (clamped to a
// valid row, non-decreasing in r for the buffer form); kfeat is the number
// of K features (A rows carry 4 bytes per feature, B rows 2).
template <int BM, int BN, int SB, int NS, int WGM = 2, int WGN = 2, bool BUF = true,
          class RowA, class RowB>
__device__ __forceinline__ void tile_product_hl(const RowA& rowA, const RowB& rowB, int kfeat,
                                                char* lds,
                                                f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  using TL = DmaTileHL<BM, BN, SB, NS, WGM, WGN>;
  const char* pa[TL::kLdA];
  const char* pb[TL::kLdB];
  uint32_t va[TL::kLdA], vb[TL::kLdB];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < TL::kLdA; ++i) {
    const int r = (wave * TL::kLdA + i) * TL::kRowsPerKBA + lane / TL::kSlotsA;
    pa[i] = rowA(r) + (((lane % TL::kSlotsA) ^ swz<SB>(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < TL::kLdB; ++i) {
    const int r = (wave * TL::kLdB + i) * TL::kRowsPerKBB + lane / TL::kSlotsB;
    pb[i] = rowB(r) + (((lane % TL::kSlotsB) ^ swz<TL::SBB>(r)) << 4);
  }
  __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
  __amdgpu_buffer_rsrc_t rb = ra;
  if constexpr (BUF) {
    auto uniform = [](const char* p) {
      const uint64_t u = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
      return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
    };
    const char* a0 = uniform(rowA(0));
    const char* b0 = uniform(rowB(0));
    const int na = __builtin_amdgcn_readfirstlane(int(rowA(BM - 1) - a0) + 4 * kfeat);
    const int nb = __builtin_amdgcn_readfirstlane(int(rowB(BN - 1) - b0) + 2 * kfeat);
#pragma unroll
    for (int i = 0; i < TL::kLdA; ++i) va[i] = uint32_t(pa[i] - a0);
#pragma unroll
    for (int i = 0; i < TL::kLdB; ++i) vb[i] = uint32_t(pb[i] - b0);
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a0), 0, na, 0x00020000);
    rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b0), 0, nb, 0x00020000);
  }
  gemm_mainloop_dma_hl<BM, BN, SB, NS, WGM, WGN, BUF>(pa, pb, va, vb, ra, rb, 4 * kfeat / SB, lds,
                                                      acc);
}

// Write the accumulators of the waves whose wave-row is `part` (or of every
// wave when part < 0) to LDS as a row-major fp32 tile with row stride `ld`
// floats; tile row 0 is the first row of that wave-row (or of the
// workgroup).  With ld % 64 == 8 the two half-waves (rows 4 apart) land on
// disjoint banks.  Callers synchronise before reading it back.
template <int BM, int BN, int WGM = 2, int WGN = 2>
__device__ __forceinline__ void acc_to_lds(const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                           float* tile, int ld, int part = -1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  if (part >= 0 && wm != part) return;
  const int row0 = part >= 0 ? 0 : wm * (BM / WGM);
#pragma unroll
  for (int i = 0; i < BM / WGM / 32; ++i)
#pragma unroll
    for (int j = 0; j < BN / WGN / 32; ++j) {
      const int col = wn * (BN / WGN) + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(row0 + i * 32 + mfma32_row(r, lane)) * ld + col] = acc[i][j][r];
    }
}

// ---------------------------------------------------------------------------
template <typename E, int BM, int BN, int SB, int NS, int WGM = 2, int WGN = 2>
constexpr int mainloop_lds() {
  return sizeof(E) == 2 ? DmaTile<BM, BN, SB, NS, WGM, WGN>::kLds : Tile<E, BM, BN>::kLds;
}

// One workgroup tile of C = A * B^T: the bf16 path runs the LDS-DMA ring
// (SB bytes of K per stage, NS stages), the fp32 path the register-staged
// loop.  rowA(r) / rowB(r) return the first byte of tile-local row r
// (clamped to a valid row); kbytes is the contraction length in bytes.
// BUF (bf16 only): the buffer form of the DMA, whose resources start at the
// tile's row 0 and reach its last row plus kbytes.  It needs rowA / rowB
// non-decreasing in r and that reach below 2^31 bytes; the host picks the
// global form where a tile of kv rows could span more.
template <typename E, int BM, int BN, int SB, int NS, int WGM = 2, int WGN = 2, bool BUF = true,
          class RowA, class RowB>
__device__ __forceinline__ void tile_product(const RowA& rowA, const RowB& rowB, int kbytes,
                                             char* lds,
                                             f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  if constexpr (sizeof(E) == 2) {
    using TL = DmaTile<BM, BN, SB, NS, WGM, WGN>;
    const char* pa[TL::kLdA];
    const char* pb[TL::kLdB];
    uint32_t va[TL::kLdA], vb[TL::kLdB];
#pragma unroll
    for (int i = 0; i < TL::kLdA; ++i) {
      const int r = dma_row<TL, SB>(i, TL::kLdA);
      pa[i] = rowA(r) + dma_slot<TL, SB>(r);
    }
#pragma unroll
    for (int i = 0; i < TL::kLdB; ++i) {
      const int r = dma_row<TL, SB>(i, TL::kLdB);
      pb[i] = rowB(r) + dma_slot<TL, SB>(r);
    }
    // (unused by the global form)
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
    __amdgpu_buffer_rsrc_t rb = ra;
    if constexpr (BUF) {
      // wave-uniform by construction; readfirstlane keeps them in SGPRs
      auto uniform = [](const char* p) {
        const uint64_t u = reinterpret_cast<uint64_t>(p);
        const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
        return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
      };
      const char* a0 = uniform(rowA(0));
      const char* b0 = uniform(rowB(0));
      const int na = __builtin_amdgcn_readfirstlane(int(rowA(BM - 1) - a0) + kbytes);
      const int nb = __builtin_amdgcn_readfirstlane(int(rowB(BN - 1) - b0) + kbytes);
#pragma unroll
      for (int i = 0; i < TL::kLdA; ++i) va[i] = uint32_t(pa[i] - a0);
#pragma unroll
      for (int i = 0; i < TL::kLdB; ++i) vb[i] = uint32_t(pb[i] - b0);
      ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(a0), 0, na, 0x00020000);
      rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b0), 0, nb, 0x00020000);
    }
    gemm_mainloop_dma<BM, BN, SB, NS, WGM, WGN, BUF>(pa, pb, va, vb, ra, rb, kbytes / SB, lds, acc);
  } else {
    static_assert(WGM == 2 && WGN == 2, "the fp32 loop runs a 2 x 2 wave grid");
    using TL = Tile<E, BM, BN>;
    const int srow = threadIdx.x >> 3, scol = (threadIdx.x & 7) * 16;
    const char* pa[TL::kLdA];
    const char* pb[TL::kLdB];
#pragma unroll
    for (int i = 0; i < TL::kLdA; ++i) pa[i] = rowA(srow + 32 * i) + scol;
#pragma unroll
    for (int i = 0; i < TL::kLdB; ++i) pb[i] = rowB(srow + 32 * i) + scol;
    gemm_mainloop<E, BM, BN>(pa, pb, kbytes / TL::kStage, lds, acc);
  }
}

}  // namespace rkv
