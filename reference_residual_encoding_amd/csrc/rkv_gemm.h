// MFMA main loop shared by every contraction of the encode path.
//
// One 256-thread workgroup computes a BM x BN tile of C = A * B^T where every
// row of A and of B is K-contiguous in HBM (the "NT" form: token rows of kv,
// packed weight rows, reference rows all have their contraction index
// innermost).  The four waves form a 2 x 2 grid; wave (wm, wn) owns the
// (BM/2) x (BN/2) sub-tile as (BM/64) x (BN/64) fragments of 32 x 32 fp32
// accumulators.
//
//  - bf16 operands use v_mfma_f32_32x32x16_bf16 (products exact, fp32 sums);
//    fp32 operands use v_mfma_f32_32x32x2_f32.  Both write the same 32 x 32
//    accumulator layout, so every epilogue serves both element types.
//  - K advances 128 bytes per stage (64 bf16 or 32 fp32).  Stages are
//    double-buffered in LDS; each thread stages 16-byte chunks through
//    registers, so the next stage's global loads are in flight while the
//    current stage feeds the matrix cores.  One barrier per stage.
//  - LDS rows are padded by 16 bytes: the 32 lanes of a half-wave that read
//    32 consecutive rows at the same K offset hit distinct banks.
//
// Callers hand in, per thread, the address of the 16-byte chunk it stages for
// each of its rows (row = tid/8 + 32*i, chunk = tid%8); rows past the end of
// a matrix must point at any valid row (their results are masked by the
// epilogue).
#pragma once
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

// Write a workgroup's accumulators to LDS as a row-major fp32 tile with row
// stride `ld` floats.  With ld % 64 == 8 the two half-waves (rows 4 apart)
// land on disjoint banks.  Callers synchronise before reading it back.
template <int BM, int BN>
__device__ __forceinline__ void acc_to_lds(const f32x16 (&acc)[BM / 64][BN / 64], float* tile,
                                           int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int j = 0; j < BN / 64; ++j) {
      const int col = wn * (BN / 2) + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(wm * (BM / 2) + i * 32 + mfma32_row(r, lane)) * ld + col] = acc[i][j][r];
    }
}

}  // namespace rkv
