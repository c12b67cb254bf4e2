// HIP kernels of the ResidualKV cache-write path for gfx950 (MI355X).
//
// Method: the ResidualKV reading notes, "ResidualKV：基于参考向量与残差的 KV Cache
// 压缩" (notes on arXiv 2602.08005v2), cited as [RKV] with the notes' own
// section numbers.
//
// Encode pipeline (one stream, in this order):
//   pack      W1|W2 -> Wp [2 d_ff][C] (columns of W1 and W2 interleaved in
//             blocks of 32 so one lane holds x*W1 and x*W2 of the same
//             column), W3 -> W3p [d_c][d_ff] (K-contiguous rows).
//   norms     reference rows copied into a compact block, and ||kv_j||^2.
//   dist      distance contraction token x reference on the matrix cores,
//             fused with a running top-KL per token and reference chunk
//             ([RKV] §2.2 retrieval equation).  Distances are ranked as
//             ||kv_j||^2 - 2 kv_t . kv_j, which orders references exactly
//             as ||kv_t - kv_j||^2 does (the dropped ||kv_t||^2 is the same
//             for every candidate of token t).
//   merge     per token: merge chunk lists, keep k_t = min(k, |pool|),
//             write ref_idx sorted by position.
//   proj      P = R [W1|W2] for the reference rows, fp32.
//   swiglu    U = kv_t [W1|W2] for non-reference tokens; epilogue forms the
//             mean branch from P (m_t [W1|W2] = mean_j kv_j [W1|W2] because
//             the first layer is linear and bias-free, [RKV] §2.3) and writes
//             delta_h = Swish(u1)*u2 - Swish(mean u1)*mean u2.
//   w3        z = delta_h W3: since W3 is linear, f_c(kv) - f_c(m) equals
//             (h(kv) - h(m)) W3 ([RKV] §2.3).  bf16 runs feed delta_h as a
//             hi + lo pair of bf16 per feature (every 8 features: 16 bytes
//             of hi, then 16 of lo), each W3 fragment multiplying both, so
//             the product keeps ~16 mantissa bits of delta_h.  The epilogue
//             runs the per-token group min-max quantiser ([RKV] §2.4) and
//             writes the record.
//   (the merge writes the all-zero records of reference tokens)
// The read side is one kernel: gather-dequantise over an index list.
#include "rkv_device.h"
#include "rkv_gemm.h"
#include "rkv_internal.h"
#include "rkv_quant.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

namespace rkv {

namespace {

// Workgroup tiles (4 waves in a 2 x 2 grid, each wave a quarter of the
// tile) and, for bf16, the DMA ring: SB bytes of K per stage, NS stages.
// reference projection: BM references x BN columns of [W1|W2] per workgroup
// token projection + SwiGLU, and the W3 product + quantiser: bf16 runs use
// 256 x 256 tiles on 8 waves (2 x 4, one workgroup per CU, a 2-stage ring
// of 128-byte K slices); fp32 runs keep the 4-wave register-staged loop
template <typename E> struct SwCfg {
  static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WGM = 2, WGN = 4;
  static constexpr int kThreads = 64 * WGM * WGN;
};
template <> struct SwCfg<float> {
  static constexpr int BM = 256, BN = 128, SB = 128, NS = 2, WGM = 2, WGN = 2;
  static constexpr int kThreads = 64 * WGM * WGN;
};
// the W3 product streams delta_h from beyond L2 as (hi, lo) pairs against
// W3 rows that hold each value once (gemm_mainloop_dma_hl): three stages of
// 128 bytes of delta_h and 64 bytes of W3 per row
template <typename E> struct W3Cfg {
  static constexpr int BM = 256, BN = 256, SB = 128, NS = 3, WGM = 2, WGN = 4, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
};
template <> struct W3Cfg<float> {
  static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WGM = 2, WGN = 2, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
};
// bf16 W3 tiles for shapes whose 256 x 256 tiles would leave most CUs idle:
// 128 x 128 on 4 waves, the same ring, two workgroups per CU (g <= 64
// divides 128, so groups stay whole)
struct W3CfgNarrow {
  static constexpr int BM = 128, BN = 128, SB = 128, NS = 3, WGM = 2, WGN = 2, kMinWaves = 2;
  static constexpr int kThreads = 64 * WGM * WGN;
};
                                                                 // difference, 2 WGs per CU
// a workgroup tile of a contraction: BM x BN outputs on a WGM x WGN wave
// grid, SB bytes of K per ring stage, NS stages
template <int BM_, int BN_, int SB_, int NS_, int WGM_, int WGN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, SB = SB_, NS = NS_, WGM = WGM_, WGN = WGN_;
  static constexpr int kThreads = 64 * WGM * WGN;
};
// distance contraction: BM references (a chunk) x BN tokens per workgroup.
// Proj is the tile of the reference projection, whose workgroups run at the
// end of the same launch: the distance tile's wave grid, on a ring that fits
// its LDS.  kMinWaves: waves per SIMD the registers must leave room for.
// bf16 runs take the wide tiles (8 waves, one workgroup per CU), or the
// narrow ones (4 waves on 128 tokens and a three-stage ring of 64-byte
// slices, two workgroups per CU, so that one scans its lists while the other
// runs its main loop) where the host finds the wide ones short of work, on
// chunks of 128 references where the wide tiles would not fill two rounds.
// Both take 256-reference chunks (measured 1.9% faster per step than 192 at
// llama8b_T32k, 1% at qwen7b_like_B2_T32k, since the projection tiles fill
// the last round of items).
template <typename E> struct DistCfg {
  static constexpr int BM = 256, BN = 256, SB = 128, NS = 2, WGM = 2, WGN = 4, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
  using Proj = TileCfg<256, 256, 128, 2, WGM, WGN>;
};
struct DistCfgNarrow {
  static constexpr int BM = 256, BN = 128, SB = 64, NS = 3, WGM = 2, WGN = 2, kMinWaves = 2;
  static constexpr int kThreads = 64 * WGM * WGN;
  using Proj = TileCfg<256, 128, 64, 3, WGM, WGN>;
};
template <> struct DistCfg<float> {
  static constexpr int BM = 128, BN = 256, SB = 128, NS = 2, WGM = 2, WGN = 2, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
  using Proj = TileCfg<128, 128, 128, 2, WGM, WGN>;
};
struct DistCfgShort {
  static constexpr int BM = 128, BN = 128, SB = 64, NS = 3, WGM = 2, WGN = 2, kMinWaves = 2;
  static constexpr int kThreads = 64 * WGM * WGN;
  using Proj = TileCfg<128, 128, 64, 3, WGM, WGN>;
};
// the smallest chunk of any tiling: the partial lists' buffer is sized for it
constexpr int kMinChunk = 128;
static_assert(DistCfgShort::BM == kMinChunk && DistCfg<float>::BM == kMinChunk &&
              DistCfg<uint16_t>::BM >= kMinChunk && DistCfgNarrow::BM >= kMinChunk,
              "no tiling cuts more chunks than kMinChunk gives");
constexpr int kEpiLd(int bn) { return bn + 8; }  // padded fp32 row of an LDS-staged tile


// ------------------------------------------------------------------ packing
// dst[map(c) * ld + r] = src[r * cols + c] for the weight matrices, one
// launch for all three.  map: 0 identity, 1 W1 slot 64*(c/32) + c%32, 2 W2
// slot 64*(c/32) + 32 + c%32.  A workgroup moves one 64 x 64 tile with
// 16-byte loads and stores (rows and columns are multiples of 32).
struct PackJob {
  const void* src;
  void* dst;
  int rows, cols, ld, mode, tiles_c, first;
};
struct PackJobs { PackJob j[3]; };

template <typename E>
constexpr int kPackLdt = 64 + 16 / int(sizeof(E));       // padded tile row (keeps 16-byte alignment)

template <typename E>
__device__ __forceinline__ void pack_tile(const PackJobs& jobs, int w, E (*tile)[kPackLdt<E>]) {
  constexpr int V = 16 / int(sizeof(E));                 // elements per 16 bytes
  const int ji = w >= jobs.j[2].first ? 2 : (w >= jobs.j[1].first ? 1 : 0);
  const PackJob& J = jobs.j[ji];
  const int tr = (w - J.first) / J.tiles_c, tc = (w - J.first) % J.tiles_c;
  const int r0 = tr * 64, c0 = tc * 64;
  const E* src = static_cast<const E*>(J.src);
  E* dst = static_cast<E*>(J.dst);
  constexpr int kVecRow = 64 / V;                        // 16-byte vectors per tile row
  for (int u = threadIdx.x; u < 64 * kVecRow; u += 256) {
    const int rr = u / kVecRow, cv = (u % kVecRow) * V;
    if (r0 + rr < J.rows && c0 + cv < J.cols)
      *reinterpret_cast<u32x4*>(&tile[rr][cv]) =
          *reinterpret_cast<const u32x4*>(src + size_t(r0 + rr) * J.cols + c0 + cv);
  }
  __syncthreads();
  for (int u = threadIdx.x; u < 64 * kVecRow; u += 256) {
    const int c = u / kVecRow, rv = (u % kVecRow) * V;   // output: column c, rows rv .. rv+V-1
    const int cg = c0 + c, rg = r0 + rv;
    if (cg >= J.cols || rg >= J.rows) continue;
    const int n = J.mode == 0 ? cg : 64 * (cg >> 5) + (J.mode == 2 ? 32 : 0) + (cg & 31);
    E v[V];
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = tile[rv + e][c];
    *reinterpret_cast<u32x4*>(dst + size_t(n) * J.ld + rg) = *reinterpret_cast<const u32x4*>(&v[0]);
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_pack_weights(PackJobs jobs) {
  __shared__ __attribute__((aligned(16))) E tile[64][kPackLdt<E>];
  pack_tile<E>(jobs, blockIdx.x, tile);
}

// ------------------------------------------------------------------ schedule
// Device copies of the reference schedule ([RKV] §2.6), one per call (every
// sequence shares it): rpos[j] = position of the j-th reference, nrp[q] =
// position of the q-th non-reference token, tab[t] = ~j for the j-th
// reference, else q.  The host computes the schedule exactly; the device
// copy comes from the closed form (fixed stride) or from the host's
// positions carried in kernel arguments, so no host buffer is involved.
// Tables for the 256 positions of block `blk`.  Fixed stride after the
// sinks (rpos_in == null): every table has a closed form, and rpos is
// written too; otherwise the positions rpos_in (already on the device) are
// searched.
struct SchedArgs {
  const int* rpos_in;
  int* rpos;
  int* tab;
  int* nrp;
  int nref, T, s0, n_sink;
};
__device__ __forceinline__ void sched_block(const SchedArgs& a, int blk) {
  const int t = blk * 256 + threadIdx.x;
  if (t >= a.T) return;
  int before;
  bool ref;
  if (a.rpos_in == nullptr) {
    if (t < a.nref) a.rpos[t] = t < a.n_sink ? t : a.n_sink + (t - a.n_sink) * a.s0;
    const int u = t - a.n_sink;
    ref = u < 0 || u % a.s0 == 0;
    before = u < 0 ? t : a.n_sink + (u + a.s0 - 1) / a.s0;   // references before t
  } else {
    int lo = 0, hi = a.nref;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.rpos_in[mid] < t) lo = mid + 1; else hi = mid;
    }
    ref = lo < a.nref && a.rpos_in[lo] == t;
    before = lo;
  }
  a.tab[t] = ref ? ~before : t - before;
  if (!ref) a.nrp[t - before] = t;
}

__global__ __launch_bounds__(256) void k_sched_fixed(int* __restrict__ rpos, int nref, int T,
                                                     int s0, int n_sink, int* __restrict__ tab,
                                                     int* __restrict__ nrp) {
  // Fixed stride after the sinks: every table has a closed form.
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (t < nref) rpos[t] = t < n_sink ? t : n_sink + (t - n_sink) * s0;
  const int u = t - n_sink;
  const bool ref = u < 0 || u % s0 == 0;
  const int before = u < 0 ? t : n_sink + (u + s0 - 1) / s0;   // references before t
  tab[t] = ref ? ~before : t - before;
  if (!ref) nrp[t - before] = t;
}

constexpr int kPosChunk = 960;
struct PosChunk {
  int first, count;
  int pos[kPosChunk];
};

__global__ __launch_bounds__(256) void k_sched_chunk(int* __restrict__ rpos, PosChunk c) {
  for (int i = threadIdx.x; i < c.count; i += 256) rpos[c.first + i] = c.pos[i];
}

__global__ __launch_bounds__(256) void k_sched_tables(const int* __restrict__ rpos, int nref,
                                                      int T, int* __restrict__ tab,
                                                      int* __restrict__ nrp) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = nref;                                 // references before t
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rpos[mid] < t) lo = mid + 1; else hi = mid;
  }
  const bool ref = lo < nref && rpos[lo] == t;
  tab[t] = ref ? ~lo : t - lo;
  if (!ref) nrp[t - lo] = t;
}

// ------------------------------------------------------------------ references
// Copy the reference rows (positions j*s of each sequence) into a compact
// [B*nref][C] block, which the distance and projection contractions stream
// (the references sit a whole stride apart in kv), and compute ||kv_j||^2;
// the row after the block is written all zero (the distance tiles read it
// for rows no token of a tile may use).
// A reference token is stored as it is ([RKV] §2.4): its ref_idx row is all
// -1 and, when a record is given, its record (codes, scale, zmin, z) is all
// zero; one wave writes each with coalesced stores.
struct RefArgs {
  const char* kv;
  char* refs;
  float* ysq;
  int32_t* ref_idx;
  uint8_t* codes;
  uint16_t* scale;
  uint16_t* zmin;
  float* z;
  SchedView sv;                                          // positions of the references
  int B, T, C, nref, k, cb, ng, d_c, fp8;
};
template <typename E>
__device__ __forceinline__ void ref_rows(const RefArgs& a, int blk) {
  const char* __restrict__ kv = a.kv;
  char* __restrict__ refs = a.refs;
  int32_t* __restrict__ ref_idx = a.ref_idx;
  uint8_t* __restrict__ codes = a.codes;
  uint16_t* __restrict__ scale = a.scale;
  uint16_t* __restrict__ zmin = a.zmin;
  float* __restrict__ z = a.z;
  const int T = a.T, C = a.C, nref = a.nref, k = a.k, cb = a.cb, ng = a.ng, d_c = a.d_c;
  const int fp8 = a.fp8;
  const int wid = blk * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= a.B * nref) {
    if (wid == a.B * nref) {                             // the zero row after the block
      char* zr = refs + size_t(wid) * C * sizeof(E);
      for (size_t o = size_t(lane) * 16; o < size_t(C) * sizeof(E); o += 64 * 16)
        *reinterpret_cast<uint4*>(zr + o) = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  const int b = wid / nref, j = wid % nref;
  const size_t rec = size_t(b) * T + size_t(ref_position(a.sv, j));   // the reference token's row
  const size_t rowb = size_t(C) * sizeof(E);
  const char* src = kv + rec * rowb;
  char* dst = refs + size_t(wid) * rowb;
  // the row's first 4 KiB requested before the record's stores, every load
  // of a batch before any is used (bytes past the row re-read byte 0)
  constexpr int U = 4;
  uint4 w[U];
  auto request = [&](size_t o0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t o = o0 + size_t(u) * 1024 + size_t(lane) * 16;
      w[u] = *reinterpret_cast<const uint4*>(src + (o < rowb ? o : 0));
    }
  };
  request(0);
  for (int i = lane; i < k; i += 64) ref_idx[rec * k + i] = -1;
  if (codes) {
    for (int o = lane * 4; o < cb; o += 256) *reinterpret_cast<uint32_t*>(codes + rec * cb + o) = 0u;
    for (int i = lane; i < ng; i += 64) { scale[rec * ng + i] = 0; zmin[rec * ng + i] = 0; }
    if (z)
      for (int i = lane * 4; i < d_c; i += 256)
        *reinterpret_cast<float4*>(z + rec * d_c + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc = 0.0f;
  for (size_t o0 = 0; o0 < rowb; o0 += U * 1024) {
    if (o0 > 0) request(o0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const size_t o = o0 + size_t(v) * 1024 + size_t(lane) * 16;
      if (o >= rowb) break;
      uint32_t u[4] = {w[v].x, w[v].y, w[v].z, w[v].w};
      if (fp8) {                                         // the values the FP8 store holds
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (sizeof(E) == 2) {
            const float lo = fp8_round(__uint_as_float(u[e] << 16));
            const float hi = fp8_round(__uint_as_float(u[e] & 0xFFFF0000u));
            u[e] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);  // exact in bf16
          } else {
            u[e] = __float_as_uint(fp8_round(__uint_as_float(u[e])));
          }
        }
      }
      *reinterpret_cast<uint4*>(dst + o) = make_uint4(u[0], u[1], u[2], u[3]);
      if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xFFFF0000u);
          acc = fmaf(lo, lo, acc);
          acc = fmaf(hi, hi, acc);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = __uint_as_float(u[e]);
          acc = fmaf(f, f, acc);
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) a.ysq[wid] = acc;
}

// One launch for the set-up of an encode, three independent parts by block
// range: weight repacking (pack tiles), schedule tables (256 positions per
// block) and the reference rows (4 per block).
template <typename E>
__global__ __launch_bounds__(256) void k_setup(PackJobs jobs, int n_pack, SchedArgs sa, int n_tab,
                                               RefArgs ra) {
  __shared__ __attribute__((aligned(16))) E tile[64][kPackLdt<E>];
  int w = blockIdx.x;
  if (w < n_pack) {
    pack_tile<E>(jobs, w, tile);
    return;
  }
  w -= n_pack;
  if (w < n_tab) {
    sched_block(sa, w);
    return;
  }
  ref_rows<E>(ra, w - n_tab);
}

// FP8 reference store ([RKV] §2.4 last paragraph): store[b][j][c] = E4M3 of
// kv[b][p_j][c], one wave per reference row, 8 coordinates per lane and
// step.  Positions come from the closed form of a fixed stride (sv), or,
// with use_chunk, from the chunk of host positions in the kernel arguments
// (references chunk.first .. chunk.first + chunk.count - 1).
template <typename E>
__global__ __launch_bounds__(256) void k_ref_store(const E* __restrict__ kv, int B, int T, int C,
                                                   SchedView sv, PosChunk chunk, int use_chunk,
                                                   int nref, uint8_t* __restrict__ store) {
  const int rows = use_chunk ? chunk.count : nref;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= B * rows) return;
  const int b = wid / rows, jj = wid % rows;
  const int j = use_chunk ? chunk.first + jj : jj;
  const int t = use_chunk ? chunk.pos[jj] : ref_position(sv, j);
  const E* src = kv + (size_t(b) * T + t) * C;
  uint8_t* dst = store + (size_t(b) * nref + j) * C;
  for (int o = lane * 8; o < C; o += 512) {
    float v[8];
    if constexpr (sizeof(E) == 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + o);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(u[e] << 16);
        v[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
      }
    } else {
      const float4 a0 = reinterpret_cast<const float4*>(src + o)[0];
      const float4 a1 = reinterpret_cast<const float4*>(src + o)[1];
      v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
      v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    }
    uint2 out;
    out.x = f32_to_fp8_e4m3(v[0]) | (f32_to_fp8_e4m3(v[1]) << 8) | (f32_to_fp8_e4m3(v[2]) << 16) |
            (f32_to_fp8_e4m3(v[3]) << 24);
    out.y = f32_to_fp8_e4m3(v[4]) | (f32_to_fp8_e4m3(v[5]) << 8) | (f32_to_fp8_e4m3(v[6]) << 16) |
            (f32_to_fp8_e4m3(v[7]) << 24);
    *reinterpret_cast<uint2*>(dst + o) = out;
  }
}

// ------------------------------------------------------------------ retrieval
// ------------------------------------------------------------------ reference projection
// One tile of P = R [W1|W2] in fp32 ([RKV] §2.2 mean eq.: the first layer of
// f_c is linear, so the mean of the chosen references' rows of P is the
// first layer applied to their mean).  R is the compact reference rows
// (M = B * nref), wp the packed [W1|W2] (N = 2 d_ff rows of C).  Tile `tile`
// of tiles_m x tiles_n, row tile fastest.
template <typename E, typename CF, bool UNPACK, typename RowOf>
__device__ __forceinline__ void ref_proj_tile_rows(const RowOf& rowof, const char* __restrict__ wp,
                                                   float* __restrict__ proj, int C, int M, int N,
                                                   int tiles_m, int tile, char* lds);

template <typename E, typename CF>
__device__ __forceinline__ void ref_proj_tile(const char* __restrict__ refs,
                                              const char* __restrict__ wp,
                                              float* __restrict__ proj, int C, int M, int N,
                                              int tiles_m, int tile, char* lds) {
  const size_t rb = size_t(C) * sizeof(E);
  ref_proj_tile_rows<E, CF, false>([&](int m) { return refs + size_t(m) * rb; }, wp, proj, C, M,
                                   N, tiles_m, tile, lds);
}

// The same tile with row m of R at rowof(m) (m < M).  The packed weights
// interleave W1 and W2 in blocks of 32 outputs (32 of W1, then the same 32
// of W2); with UNPACK the columns are stored in the order [W1 | W2].
template <typename E, typename CF, bool UNPACK, typename RowOf>
__device__ __forceinline__ void ref_proj_tile_rows(const RowOf& rowof,
                                                   const char* __restrict__ wp,
                                                   float* __restrict__ proj, int C, int M, int N,
                                                   int tiles_m, int tile, char* lds) {
  constexpr int BM = CF::BM, BN = CF::BN, WGM = CF::WGM, WGN = CF::WGN;
  constexpr int kWM = BM / WGM, kWN = BN / WGN, kTM = kWM / 32, kTN = kWN / 32;
  const int mt = tile % tiles_m, nt = tile / tiles_m;
  const int m0 = mt * BM, n0 = nt * BN;
  const size_t rowb = size_t(C) * sizeof(E);
  const int tid = threadIdx.x;
  auto rowA = [&](int r) { return rowof(min(m0 + r, M - 1)); };
  auto rowB = [&](int r) { return wp + size_t(min(n0 + r, N - 1)) * rowb; };
  f32x16 acc[kTM][kTN];
  tile_product<E, BM, BN, CF::SB, CF::NS, WGM, WGN>(rowA, rowB, int(rowb), lds, acc);
  const int lane = tid & 63, wave = tid >> 6, wm = wave / WGN, wn = wave % WGN;
#pragma unroll
  for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < kTN; ++tn) {
      const int col = n0 + wn * kWN + tn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * kWM + tm * 32 + mfma32_row(r, lane);
        if (row < M && col < N) {
          const int o = UNPACK ? ((col >> 5) & 1) * (N >> 1) + (col >> 6) * 32 + (col & 31) : col;
          proj[size_t(row) * N + o] = acc[tm][tn][r];
        }
      }
    }
}

// One workgroup: BM references (chunk c) x BN non-reference tokens (tile tt)
// of sequence b.  Every lane scans the dot products its own accumulators
// hold (its kTN tokens against its kTM*16 references, in increasing j),
// keeping a top-KL list per token; the 2*WGM lists of a token (two lane
// halves of each of the WGM waves that share its columns) are then
// combined in LDS into the KL best (d', j) of the chunk restricted to the
// causal pool, written as partial list c.
// BUF: the buffer form of the operand DMA (the host checks that a token
// tile's rows lie within 2^31 bytes).
// Workgroups n_dist and beyond compute tiles of the reference projection
// (ref_proj_tile) instead: that product reads only the compact reference
// rows and the packed weights, and after every distance item has been
// dealt its tiles fill the CUs the last round of items leaves idle.
template <typename E, typename CF, int KL, bool BUF>
__global__ __launch_bounds__(CF::kThreads, CF::kMinWaves) void k_dist_topk(
    const char* __restrict__ kv, const char* __restrict__ refs, const float* __restrict__ ysq,
    float2* __restrict__ part, int B, int T, int C, const int* __restrict__ nrp, int nref,
    int nr, int n_lists, int n_tt, int n_dist, const char* __restrict__ wp,
    float* __restrict__ proj, int proj_n, int proj_tiles_m, const char* __restrict__ zrow,
    int serp) {
  using PF = typename CF::Proj;
  constexpr int BM = CF::BM, BN = CF::BN, WGM = CF::WGM, WGN = CF::WGN;
  constexpr int kLists = 2 * WGM;                        // partial lists per token
  constexpr int kMain = mainloop_lds<E, BM, BN, CF::SB, CF::NS, WGM, WGN>();
  constexpr int kComb = BN * kLists * KL * 8;            // the lists, as (d', j) pairs
  constexpr int kProj = mainloop_lds<E, PF::BM, PF::BN, PF::SB, PF::NS, PF::WGM, PF::WGN>();
  static_assert(kProj <= (kMain > kComb ? kMain : kComb), "the projection tile fits the LDS");
  constexpr int kStaged = kMain > kComb ? kMain : kComb;
  __shared__ __attribute__((aligned(1024))) char lds[kStaged + BM * 4];
  if (int(blockIdx.x) >= n_dist) {
    ref_proj_tile<E, PF>(refs, wp, proj, C, B * nref, proj_n, proj_tiles_m,
                         int(blockIdx.x) - n_dist, lds);
    return;
  }
  float* ysq_l = reinterpret_cast<float*>(lds + kStaged);
  // Work items are the causal (token tile, reference chunk) pairs.  The
  // dispatcher deals workgroups to the 8 XCDs in turn, so workgroup w runs
  // on XCD w % 8: that XCD takes one token tile of every row of 8, g = 8m +
  // x (or, with serp, 8m + 7 - x for odd m: later tiles have longer pools,
  // so the alternation evens the XCDs' item counts), and all of their
  // chunks, one after the other, which keeps a token tile in its own L2
  // while the chunks stream past.
  // Every wave finds the item alike: its 64 lanes take 64 of the XCD's token
  // tiles at once (one load each, not a chain of dependent loads), and a
  // prefix sum of their chunk counts over the lanes locates item l.
  const int x = blockIdx.x & 7;
  const int l = blockIdx.x >> 3;
  const int lane = threadIdx.x & 63;
  int g = -1, c = -1;
  for (int m0l = 0, before = 0; 8 * m0l < B * n_tt; m0l += 64) {
    const int ml = m0l + lane;
    const int gl = 8 * ml + ((serp && (ml & 1)) ? 7 - x : x);
    int np = 0, nch = 0;
    if (gl < B * n_tt) {
      const int tt_ = gl % n_tt;
      const int ql = min(tt_ * BN + BN, nr) - 1;        // last token of the tile
      np = nrp[ql] - ql;                                 // its pool: references before it
      nch = (np + BM - 1) / BM;
    }
    int incl = nch;                                      // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int want = l - before;
    const unsigned long long hit = __ballot(want >= incl - nch && want < incl);
    if (hit) {
      const int src = __ffsll(hit) - 1;
      g = __shfl(gl, src);
      c = want - (__shfl(incl, src) - __shfl(nch, src));
      break;
    }
    before += __shfl(incl, 63);
  }
  if (c < 0) return;  // this XCD has no more items
  const int tt = g % n_tt, b = g / n_tt;
  const int n0 = tt * BN;
  const int m0 = c * BM;

  const size_t rowb = size_t(C) * sizeof(E);
  const char* base = kv + size_t(b) * T * rowb;
  const int tid = threadIdx.x;
  // the chunk's reference norms: loaded before the main loop (their latency
  // passes under the first stages' copies), published after it
  static_assert(BM <= CF::kThreads, "one norm per thread");
  const float ysq_r = tid < BM ? ysq[size_t(b) * nref + min(m0 + tid, nref - 1)] : 0.0f;
  const char* rbase = refs + size_t(b) * nref * rowb;
  // Rows of the chunk that no token of the tile may use (past the last
  // token's pool, or past the last reference) read the all-zero row after
  // the reference block (zrow, when given): their dot products are masked
  // anyway, and the matrix cores draw far less power on zero operands than
  // on a duplicated reference row.  The row lies past every reference row,
  // so the addresses stay non-decreasing in r.
  const int qlast = min(n0 + BN, nr) - 1;
  const int nvalid = zrow ? min(nrp[qlast] - qlast, nref) - m0 : BM;
  auto rowA = [&](int r) {
    return r < nvalid ? rbase + size_t(min(m0 + r, nref - 1)) * rowb : zrow;
  };
  auto rowB = [&](int r) { return base + size_t(nrp[min(n0 + r, nr - 1)]) * rowb; };
  f32x16 acc[BM / WGM / 32][BN / WGN / 32];
  tile_product<E, BM, BN, CF::SB, CF::NS, WGM, WGN, BUF>(rowA, rowB, int(rowb), lds, acc);
  if (tid < BM) ysq_l[tid] = ysq_r;
  __syncthreads();

  // Lane l of wave (wm, wn) holds in register r of fragment (i, j) the dot
  // product of token column wn*kWN + 32j + l%32 with chunk reference
  // wm*kWM + 32i + mfma32_row(r, l): for each of its tokens it sees kTM*16
  // references, in increasing j as i, then r, increase.  d' = ||y||^2 -
  // 2 x.y ranks them as the distance does ([RKV] §2.2).  Candidates outside
  // the token's causal pool (j at or past the references before its
  // position) are masked, unless the whole item lies inside every pool.
  constexpr int kWM = BM / WGM, kWN = BN / WGN, kTM = kWM / 32, kTN = kWN / 32;
  const int wave = tid >> 6, hi = lane >> 5;
  const int wm = wave / WGN, wn = wave % WGN;
  int lim[kTN];
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int q = n0 + wn * kWN + 32 * j + (lane & 31);
    lim[j] = q < nr ? nrp[q] - q - m0 : 0;               // references of this chunk in its pool
  }
  // the tile's first token has the smallest pool: the whole item is causal
  // when it covers all BM references of the chunk
  const bool full = nrp[n0] - n0 - m0 >= BM;
  float bd[kTN][KL];
  int bi[kTN][KL];
#pragma unroll
  for (int j = 0; j < kTN; ++j)
#pragma unroll
    for (int i = 0; i < KL; ++i) { bd[j][i] = __builtin_inff(); bi[j][i] = 0x7fffffff; }
  auto scan = [&](auto masked_c) {
    constexpr bool kMasked = decltype(masked_c)::value;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        // four consecutive references: rows base .. base + 3 of the chunk
        const int base = wm * kWM + 32 * i + 8 * r4 + 4 * hi;
        const float4 y4 = *reinterpret_cast<const float4*>(ysq_l + base);
        const float yv[4] = {y4.x, y4.y, y4.z, y4.w};
        float dd[kTN][4];
        bool use = false;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float d = yv[u] - 2.0f * acc[i][j][4 * r4 + u];
            dd[j][u] = (!kMasked || base + u < lim[j]) ? d : __builtin_inff();
          }
          // a candidate not below the current KL-th best changes nothing (a
          // tie arrives with the larger j)
          const float mn = fminf(fminf(dd[j][0], dd[j][1]), fminf(dd[j][2], dd[j][3]));
          use |= mn < bd[j][KL - 1];
        }
        // a group no lane of the wave can use is skipped whole; otherwise the
        // lane's tokens take their candidates in turn (independent chains)
        if (__any(use)) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < kTN; ++j) topk_push<KL>(bd[j], bi[j], dd[j][u], m0 + base + u);
        }
      }
  };
  if (full)
    scan(std::false_type{});
  else
    scan(std::true_type{});

  // Combine: every lane publishes its lists (slot wm*2 + hi of its
  // tokens), then one thread per token merges the kLists lists by (d, j).
  float2* xl = reinterpret_cast<float2*>(lds);           // [BN][kLists][KL]
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int t = wn * kWN + 32 * j + (lane & 31);
    float2* dst = xl + (t * kLists + wm * 2 + hi) * KL;
#pragma unroll
    for (int i = 0; i < KL; ++i) dst[i] = make_float2(bd[j][i], __int_as_float(bi[j][i]));
  }
  __syncthreads();
  for (int t = tid; t < BN; t += CF::kThreads) {
    const int q = n0 + t;
    if (q >= nr) continue;
    float md[KL];
    int mi[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) { md[i] = __builtin_inff(); mi[i] = 0x7fffffff; }
#pragma unroll
    for (int o = 0; o < kLists; ++o) {                   // each list in ascending (d, j)
      float ld[KL];
      int li[KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        const float2 v = xl[(t * kLists + o) * KL + i];
        ld[i] = v.x;
        li[i] = __float_as_int(v.y);
      }
      merge_sorted_lex<KL>(md, mi, ld, li);
    }
    float2* out = part + ((size_t(b) * n_lists + c) * nr + q) * KL;
#pragma unroll
    for (int i = 0; i < KL; ++i) out[i] = make_float2(md[i], __int_as_float(mi[i]));
  }
}

// Per non-reference token: merge the partial lists, keep k_t = min(k, pool
// size) references ([RKV] §2.1), write their positions in ascending order,
// -1 pads.  The lists cover disjoint reference sets; the merge orders by
// (d, j), so equal distances keep the smaller position whatever order the
// lists come in.  (Reference tokens' all -1 rows and zero records are
// written by the set-up kernel: references are stored as they are, [RKV]
// §2.4.)  kMergeLanes consecutive lanes share a token: lane s merges lists
// s, s + 4, ..., two at a time with both in flight, then the lanes' lists
// are merged by a butterfly over the four, and the first writes the result;
// every list is in ascending (d, j) order, so each step merges two sorted
// lists (merge_sorted_lex).
constexpr int kMergeLanes = 4;

template <int KL>
__global__ __launch_bounds__(256) void k_topk_merge(const float2* __restrict__ part,
                                                     int32_t* __restrict__ ref_idx, int B, int T,
                                                     const int* __restrict__ tab,
                                                     const int* __restrict__ rpos, int k, int nr,
                                                     int n_lists, int chunk,
                                                     int* __restrict__ selj) {
  const long gid = long(blockIdx.x) * 256 + threadIdx.x;
  const long tok = gid / kMergeLanes;
  const int sub = int(gid % kMergeLanes);
  // every lane stays to the butterfly; lanes past the last token, and the
  // lanes of a reference token, merge nothing and write nothing
  const bool in = tok < long(B) * T;
  const int b = in ? int(tok / T) : 0, t = in ? int(tok % T) : 0;
  const int q = tab[t];
  const bool enc = in && q >= 0;
  const int npool = enc ? t - q : 0;
  const int kt = min(k, npool);
  const int nch = (npool + chunk - 1) / chunk;          // lists that cover the pool
  float bd[KL];
  int bi[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) { bd[i] = __builtin_inff(); bi[i] = 0x7fffffff; }
  const float2* p = part + (size_t(b) * n_lists * nr + max(q, 0)) * KL;
  const size_t cstride = size_t(nr) * KL;
  for (int c0 = sub; c0 < nch; c0 += 2 * kMergeLanes) {
    // lists c0 and c0 + 4; one past the last re-reads the last and enters
    // as padding
    float4 v[2][KL / 2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float4* src =
          reinterpret_cast<const float4*>(p + min(c0 + u * kMergeLanes, nch - 1) * cstride);
#pragma unroll
      for (int h = 0; h < KL / 2; ++h) v[u][h] = src[h];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {                        // each list in ascending (d, j)
      const bool live = c0 + u * kMergeLanes < nch;
      float ld[KL];
      int li[KL];
#pragma unroll
      for (int h = 0; h < KL / 2; ++h) {
        ld[2 * h] = live ? v[u][h].x : __builtin_inff();
        li[2 * h] = live ? __float_as_int(v[u][h].y) : 0x7fffffff;
        ld[2 * h + 1] = live ? v[u][h].z : __builtin_inff();
        li[2 * h + 1] = live ? __float_as_int(v[u][h].w) : 0x7fffffff;
      }
      merge_sorted_lex<KL>(bd, bi, ld, li);
    }
  }
#pragma unroll
  for (int off = 1; off < kMergeLanes; off <<= 1) {
    float od[KL];
    int oi[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) { od[i] = __shfl_xor(bd[i], off); oi[i] = __shfl_xor(bi[i], off); }
    merge_sorted_lex<KL>(bd, bi, od, oi);
  }
  if (!enc || sub != 0) return;
  int32_t* out = ref_idx + tok * k;
  int sel[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) sel[i] = i < kt ? bi[i] : 0x7fffffff;
#pragma unroll
  for (int i = 1; i < KL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const int a = sel[j - 1], c2 = sel[j];
      sel[j - 1] = min(a, c2);
      sel[j] = max(a, c2);
    }
#pragma unroll
  for (int i = 0; i < KL; ++i)
    if (i < k) out[i] = i < kt ? rpos[sel[i]] : -1;
  // the same choice as reference indices, for the SwiGLU's mean branch
  int4* sj = reinterpret_cast<int4*>(selj + (size_t(b) * nr + q) * KL);
#pragma unroll
  for (int h = 0; h < KL / 4; ++h)
    sj[h] = make_int4(4 * h + 0 < kt ? sel[4 * h + 0] : -1, 4 * h + 1 < kt ? sel[4 * h + 1] : -1,
                      4 * h + 2 < kt ? sel[4 * h + 2] : -1, 4 * h + 3 < kt ? sel[4 * h + 3] : -1);
}

// ------------------------------------------------------------------ Swish
// the value lane l ^ 1 holds (DPP quad permutation 1, 0, 3, 2)
__device__ __forceinline__ uint32_t lane_xor1(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float silu_fast(float x) {
  // x * sigmoid(x) with the hardware exp2 and reciprocal (about 1e-7
  // relative, far inside the latent tolerance)
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * x));
}

// ------------------------------------------------------------------ SwiGLU difference
// U = kv_t [W1|W2] for a tile of kSwBM non-reference tokens x kSwBN columns
// of Wp, then per (token, d_ff feature f)
//   delta_h = Swish(u1) * u2 - Swish(mean_j P_j,1) * mean_j P_j,2,
// where P = R [W1|W2] holds the projected references and j runs over the
// token's k_t chosen references: m_t [W1|W2] = mean_j kv_j [W1|W2] because
// the first layer of f_c is linear and bias-free ([RKV] §2.2 mean eq.,
// §2.3).  delta_h goes to row Q of dh, 4 bytes per feature: for bf16 runs
// a (hi, lo) bf16 pair, each granule of 8 features as 16 bytes of hi values
// then 16 bytes of lo values (the A layout of gemm_mainloop_dma_hl); fp32
// otherwise, feature f at float index Q*d_ff + f.
template <typename E, int KL, bool BUF, bool STREAM>
__global__ __launch_bounds__(SwCfg<E>::kThreads) void k_swiglu(const char* __restrict__ kv,
                                                const char* __restrict__ wp,
                                                const float* __restrict__ proj,
                                                uint32_t proj_bytes,
                                                const int* __restrict__ selj,
                                                char* __restrict__ dh, int T, int C,
                                                const int* __restrict__ nrp, int nref, int nr,
                                                int d_ff, int M, int col_order) {
  using CF = SwCfg<E>;
  constexpr int BM = CF::BM, BN = CF::BN, WGM = CF::WGM, WGN = CF::WGN, NT = CF::kThreads;
  constexpr int kMain = mainloop_lds<E, BM, BN, CF::SB, CF::NS, WGM, WGN>();
  constexpr int kLdh = BN / 2 + 8;                       // padded fp32 row of the staged h tile
  constexpr int kStaged = kMain > BM * kLdh * 4 ? kMain : BM * kLdh * 4;
  __shared__ __attribute__((aligned(1024))) char lds[kStaged + BM * KL * 4 + BM * 4];
  uint32_t* poff_lds = reinterpret_cast<uint32_t*>(lds + kStaged);  // [BM][KL] P row byte offsets
  float* inv_lds = reinterpret_cast<float*>(lds + kStaged + BM * KL * 4);  // [BM] 1 / k_t
  const int N = 2 * d_ff;
  // Row tile fastest (col_order 0): all XCDs work through one column tile of
  // Wp at a time, so every L2 holds that tile's rows of Wp and the columns of
  // P its epilogue gathers, while each token tile is read once per column
  // tile.  Column tile fastest (col_order 1): the column tiles of a token tile
  // run together, so its kv rows leave HBM about once (the host picks this
  // order when the kv rows outgrow the MALL).
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int mt = col_order ? int(blockIdx.x) / tiles_n : int(blockIdx.x) % tiles_m;
  const int nt = col_order ? int(blockIdx.x) % tiles_n : int(blockIdx.x) / tiles_m;
  const int m0 = mt * BM, n0 = nt * BN;
  const size_t rowb = size_t(C) * sizeof(E);
  const int tid = threadIdx.x;
  // Per token of the tile: the byte offsets of its reference rows of P and
  // 1/k_t (read back after the main loop, whose barriers publish them).  A
  // missing reference gets the offset 2^31, past the end of P (which is
  // smaller than 2 GiB) also after a column offset is added: the buffer load
  // below returns zero for it.
  // The chosen references' indices (one 16-byte load per 4, -1 pads) are
  // loaded before the main loop, whose first stages' copies cover their
  // latency, and turned into offsets after it.
  constexpr uint32_t kNone = 0x80000000u;
  static_assert(BM <= NT, "one token per thread");
  const int Qr = m0 + tid;
  int jr[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) jr[i] = -1;
  if (tid < BM && Qr < M) {
    const int4* sj = reinterpret_cast<const int4*>(selj + size_t(Qr) * KL);
#pragma unroll
    for (int h = 0; h < KL / 4; ++h) {
      const int4 v = sj[h];
      jr[4 * h] = v.x; jr[4 * h + 1] = v.y; jr[4 * h + 2] = v.z; jr[4 * h + 3] = v.w;
    }
  }
  auto rowA = [&](int r) {
    const int Q = min(m0 + r, M - 1);
    return kv + (size_t(Q / nr) * T + nrp[Q % nr]) * rowb;
  };
  auto rowB = [&](int r) { return wp + size_t(min(n0 + r, N - 1)) * rowb; };
  constexpr int kTM = BM / WGM / 32, kTN = BN / WGN / 32;
  f32x16 acc[kTM][kTN];
  tile_product<E, BM, BN, CF::SB, CF::NS, WGM, WGN, BUF>(rowA, rowB, int(rowb), lds, acc);
  if (tid < BM) {
    const int b = Qr / nr;
    int kt = 0;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      uint32_t off = kNone;
      if (jr[i] >= 0) {
        off = uint32_t(b * nref + jr[i]) * uint32_t(N) * 4u;      // P row of reference jr[i]
        ++kt;
      }
      poff_lds[tid * KL + i] = off;
    }
    inv_lds[tid] = 1.0f / float(max(kt, 1));
  }
  __syncthreads();

  // 2 (set-up). Four consecutive features of one row per lane: BN/8 lanes
  // per row, 16 rows per workgroup step.  Feature quad c holds W1 columns
  // n0 + 64(c/8) + 4(c%8) .. +3 of P and the W2 columns 32 further.  All
  // loads and stores are unconditional: P and the tile's rows of dh go
  // through buffer resources (an offset past the end of a range reads zero
  // and drops a store), which lets the compiler keep the loads in flight.
  // The P rows of the first row steps are requested before h is staged,
  // and each group's loads are in flight while the previous group is
  // consumed (two register buffers).
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int kQ = BN / 8;                             // feature quads per row
  static_assert(NT / kQ == 16, "16 rows per workgroup step");
  const int c = tid % kQ, row0 = tid / kQ;
  const bool colv = n0 + 64 * (c >> 3) < N;              // the quad's 64-column group exists
  const uint32_t pcol = uint32_t(n0 + 64 * (c >> 3) + 4 * (c & 7)) * 4u;
  const int f = n0 / 2 + 4 * c;
  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(proj), 0, int(proj_bytes), 0x00020000);
  const int rows = min(M - m0, BM);
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
      dh + size_t(m0) * d_ff * 4, 0, rows * d_ff * 4, 0x00020000);
  auto ld4 = [&](uint32_t off) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(prs, int(off), 0, 0));
  };
  constexpr int kRB = KL <= 4 ? 2 : 1;                   // row steps per group
  constexpr int kGroups = BM / 16 / kRB;
  static_assert(kGroups % 2 == 0, "groups alternate between two buffers");
  f4 pa1[kRB][KL], pa2[kRB][KL], pb1[kRB][KL], pb2[kRB][KL];
  auto issue = [&](int g, f4 (&q1)[kRB][KL], f4 (&q2)[kRB][KL]) {
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const uint32_t* po = poff_lds + (16 * (g * kRB + u) + row0) * KL;
#pragma unroll
      for (int q = 0; q < KL; ++q) {
        // kNone + pcol stays past the end of P; a quad past the column edge
        // reads in-range values of no use (its store is dropped)
        q1[u][q] = ld4(po[q] + pcol);
        q2[u][q] = ld4(po[q] + pcol + 128u);             // +32 floats: the x*W2 columns
      }
    }
  };
  issue(0, pa1, pa2);

  // 1. h(kv) = Swish(u1) * u2 from the accumulators into LDS.  Lane l of
  // wave (wm, wn) holds, in register r of fragment (i, j), tile row
  // wm*BM/WGM + 32i + mfma32_row(r, l) and Wp row n0 + wn*64 + 32j + l%32.
  // Wp interleaves W1 and W2 in blocks of 32, so fragment j = 0 is x*W1 and
  // j = 1 the x*W2 of the same feature: tile feature wn*32 + l%32.
  static_assert(kTN == 2 && BN / WGN == 64, "one W1/W2 fragment pair per wave");
  float* h = reinterpret_cast<float*>(lds);
  {
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        h[(wm * (BM / WGM) + 32 * i + mfma32_row(r, lane)) * kLdh + wn * 32 + (lane & 31)] =
            silu_fast(acc[i][0][r]) * acc[i][1][r];
  }
  __syncthreads();

  // 2. delta_h = h(kv) - Swish(mean u1) * mean u2 per row, stored as (hi, lo)
  // bf16 pairs (or fp32)
  auto consume = [&](int g, const f4 (&q1)[kRB][KL], const f4 (&q2)[kRB][KL]) {
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
      const int rt = 16 * (g * kRB + u) + row0;
      f4 s1 = q1[u][0], s2 = q2[u][0];
#pragma unroll
      for (int q = 1; q < KL; ++q) { s1 += q1[u][q]; s2 += q2[u][q]; }
      const float inv = inv_lds[rt];
      const f4 hk = *reinterpret_cast<const f4*>(h + rt * kLdh + 4 * c);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dl = hk[e] - silu_fast(s1[e] * inv) * (s2[e] * inv);
        w[e] = sizeof(E) == 2 ? bf16_hi_lo(dl) : __float_as_uint(dl);
      }
      // a quad past the column edge, or a row past M, lands outside the range
      if constexpr (sizeof(E) == 2) {
        // The row's 8-feature granule holds 16 bytes of hi values, then 16
        // of lo values.  Lanes c (even) and c + 1 hold its two quads: they
        // swap halves (DPP, lanes l and l ^ 1), the even lane then stores
        // the granule's hi values and the odd lane its lo values.
        const uint32_t hi01 = (w[0] & 0xFFFFu) | (w[1] << 16), hi23 = (w[2] & 0xFFFFu) | (w[3] << 16);
        const uint32_t lo01 = (w[0] >> 16) | (w[1] & 0xFFFF0000u), lo23 = (w[2] >> 16) | (w[3] & 0xFFFF0000u);
        const bool odd = c & 1;
        const uint32_t r0 = lane_xor1(odd ? hi01 : lo01), r1 = lane_xor1(odd ? hi23 : lo23);
        const u32x4 wv = odd ? u32x4{r0, r1, lo01, lo23} : u32x4{hi01, hi23, r0, r1};
        const uint32_t so =
            colv ? uint32_t(rt * d_ff + (f & ~7)) * 4u + (odd ? 16u : 0u) : kNone;
        // STREAM: non-temporal (slc), so delta_h streams out without evicting
        // the kv rows and P columns the later tiles read again
        __builtin_amdgcn_raw_buffer_store_b128(wv, drs, int(so), 0, STREAM ? 2 : 0);
      } else {
        const u32x4 wv = {w[0], w[1], w[2], w[3]};
        const uint32_t so = colv ? uint32_t(rt * d_ff + f) * 4u : kNone;
        __builtin_amdgcn_raw_buffer_store_b128(wv, drs, int(so), 0, 0);
      }
    }
  };
#pragma unroll
  for (int g = 0; g < kGroups; g += 2) {
    issue(g + 1, pb1, pb2);
    consume(g, pa1, pa2);
    if (g + 2 < kGroups) issue(g + 2, pa1, pa2);
    consume(g + 1, pb1, pb2);
  }
}

// ------------------------------------------------------------------ W3 + quantiser
// z = delta_h W3 for a tile of kW3BM non-reference tokens x kW3BN latent
// columns, then the group quantiser on the tile ([RKV] §2.4), writing the
// token's record (and z, if asked) at its place in [B][T].
template <typename E, typename CF, int BITS, int G8>
__global__ __launch_bounds__(CF::kThreads, CF::kMinWaves) void k_w3_quant(const char* __restrict__ dh,
                                                  const char* __restrict__ w3p, int K, int M,
                                                  int N, int tiles_m, int T,
                                                  const int* __restrict__ nrp, int nr,
                                                  uint8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ scale,
                                                  uint16_t* __restrict__ zmin,
                                                  float* __restrict__ z) {
  constexpr int BM = CF::BM, BN = CF::BN, WGM = CF::WGM, WGN = CF::WGN, NT = CF::kThreads;
  static_assert(WGM == 2, "the epilogue stages one wave-row (half the tile) at a time");
  static_assert(BN % 64 == 0 && (BM / 2) * (BN / 8) % NT == 0,
                "whole groups (g <= 64) per tile row; every thread takes the same units");
  constexpr int LD = kEpiLd(BN);
  constexpr int HALF = BM / 2;
  constexpr bool kHL = sizeof(E) == 2;                   // bf16: delta_h as (hi, lo) pairs
  constexpr int kMain = kHL ? DmaTileHL<BM, BN, CF::SB, CF::NS, WGM, WGN>::kLds
                            : mainloop_lds<E, BM, BN, CF::SB, CF::NS, WGM, WGN>();
  constexpr int kLdsBytes = kMain > HALF * LD * 4 ? kMain : HALF * LD * 4;
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes + BM * 4];
  int* rec_lds = reinterpret_cast<int*>(lds + kLdsBytes);  // [BM] record row b*T + t, -1 past M
  const int mt = blockIdx.x % tiles_m, nt = blockIdx.x / tiles_m;
  const int m0 = mt * BM, n0 = nt * BN;
  // K features: a delta_h row carries 4 bytes each (bf16 hi and lo, or
  // fp32), a packed W3 row one element each
  const size_t rowa = size_t(K) * 4, rowb = size_t(K) * sizeof(E);
  const int tid = threadIdx.x;
  // record row of every token of the tile: loaded before the main loop,
  // written to LDS after it (the epilogue's first barrier publishes it)
  static_assert(BM <= NT, "one token per thread");
  int rec_r = -1;
  if (tid < BM && m0 + tid < M) rec_r = ((m0 + tid) / nr) * T + nrp[(m0 + tid) % nr];
  auto rowA = [&](int r) { return dh + size_t(min(m0 + r, M - 1)) * rowa; };
  auto rowB = [&](int r) { return w3p + size_t(min(n0 + r, N - 1)) * rowb; };
  f32x16 acc[BM / WGM / 32][BN / WGN / 32];
  if constexpr (kHL)
    tile_product_hl<BM, BN, CF::SB, CF::NS, WGM, WGN>(rowA, rowB, K, lds, acc);
  else
    tile_product<E, BM, BN, CF::SB, CF::NS, WGM, WGN>(rowA, rowB, int(rowb), lds, acc);
  if (tid < BM) rec_lds[tid] = rec_r;
  float* zt = reinterpret_cast<float*>(lds);
  // 8 latent values per lane; G8 consecutive lanes hold one group (groups
  // never straddle a row or the edge N: g divides both BN and d_c)
  constexpr int kChunks = BN / 8;
  const int d_c = N;
  for (int half = 0; half < 2; ++half) {
    acc_to_lds<BM, BN, WGM, WGN>(acc, zt, LD, half);
    __syncthreads();
    for (int i = 0; i < HALF * kChunks / NT; ++i) {
      const int unit = i * NT + tid;
      const int row = unit / kChunks, ch = unit % kChunks;
      const int col = n0 + ch * 8;
      const int recr = rec_lds[half * HALF + row];
      const bool act = recr >= 0 && col < N;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = zt[row * LD + ch * 8 + e];
      const int64_t rec = recr;                                     // record row b*T + t
      const int64_t u = (rec * d_c + col) / 8;                      // flat 8-value unit
      write_record8<BITS, G8>(v, act, tid, u, codes, scale, zmin);
      if (act) {
        if (z) {
          float* zo = z + rec * d_c + col;
          *reinterpret_cast<float4*>(zo) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4*>(zo + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
    }
    __syncthreads();
  }
}

// Stand-alone quantiser (stepwise export): rows of z map one to one onto the
// records.  One wave covers 512 consecutive latent values (whole groups,
// since g divides 512); every lane owns 8 consecutive values of one group.
template <int BITS, int G8>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ z, int64_t rows,
                                                  int d_c, uint8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ scale,
                                                  uint16_t* __restrict__ zmin) {
  const int lane = threadIdx.x & 63;
  const int64_t units = rows * (d_c / 8);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t base = int64_t(blockIdx.x) * blockDim.x + (threadIdx.x & ~63); base < units;
       base += stride) {
    const int64_t u = base + lane;
    const bool act = u < units;
    float v[8];
    if (act) {
      const float4 a = *reinterpret_cast<const float4*>(z + u * 8);
      const float4 c = *reinterpret_cast<const float4*>(z + u * 8 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    write_record8<BITS, G8>(v, act, lane, u, codes, scale, zmin);
  }
}

// ------------------------------------------------------------------ restore
// Read side ([RKV] §2.5): KV^ = z~ W_d + mean of the token's stored
// references (a reference token is its own single reference, with z~ = 0),
// split into K | V, and K rotated at the token's own position ([RKV] §2.1
// note).  Two kernels: the selected records are dequantised into the A
// operand of the decoder product, then the product's epilogue adds the
// reference mean and applies the rotation.
// bf16 runs: z~ as (hi, lo) pairs against W_d rows holding each value once
// (gemm_mainloop_dma_hl), three stages of 128 bytes of z~ and 64 of W_d
template <typename E> struct RsCfg {
  static constexpr int BM = 256, BN = 256, SB = 128, NS = 3, WGM = 2, WGN = 4, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
};
template <> struct RsCfg<float> {
  static constexpr int BM = 256, BN = 128, SB = 128, NS = 2, WGM = 2, WGN = 2, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
};
// the 8-wave restore's tiles for the rows after its last whole round:
// 128 x 256, half the work of a 256 x 256 tile (measured better than 8-wave
// 128 x 128 tiles, whose rounds took about 0.9 of a wide round)
struct RsCfgTail {
  static constexpr int BM = 128, BN = 256, SB = 128, NS = 3, WGM = 2, WGN = 4, kMinWaves = 1;
  static constexpr int kThreads = 64 * WGM * WGN;
};
// bf16 restore tiles two to a CU, so that one workgroup's epilogue (mean
// loads, rotation, stores) runs beside the other's main loop: 128 x 128 on
// 4 waves, three stages (128 columns hold whole heads: D divides 128)
struct RsCfgNarrow {
  static constexpr int BM = 128, BN = 128, SB = 128, NS = 3, WGM = 2, WGN = 2, kMinWaves = 2;
  static constexpr int kThreads = 64 * WGM * WGN;
};

// z~ of each selected token as the decoder product's A row: bf16 runs store
// a (hi, lo) bf16 pair per latent, each 8 latents as 16 bytes of hi values
// then 16 of lo values (the A layout of gemm_mainloop_dma_hl), fp32 runs the
// float; zeros for reference tokens (all -1 ref_idx rows) and indices
// outside [0, B*T).  z~ is
// fmaf(q, Delta_h, m_h), as rkv_dequant_gather gives it.
// The unit at o = 0 of each row also writes the row's entry of rinfo
// ([kl + 4] ints): the stored rows of the references whose mean the restore
// adds (a reference token: its own row), 1/count as float bits, and the
// token's position, or all -1 and position -1 for an index outside
// [0, B*T), whose restored row is NaN.  FP8: the stored references are the
// E4M3 store [B][nref][C]; row of a reference position p = its index j in
// the schedule (closed form, or ~tab[p] from the schedule tables).
template <typename E, int BITS, int KL, bool FP8>
__global__ __launch_bounds__(256) void k_restore_prep(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scale,
                                                      const uint16_t* __restrict__ zmin,
                                                      const int32_t* __restrict__ idx,
                                                      int64_t n_idx, int64_t total_rows,
                                                      const int32_t* __restrict__ ref_idx, int k,
                                                      int d_c, int g,
                                                      uint32_t* __restrict__ zt, int T,
                                                      SchedView sv, const int* __restrict__ tab,
                                                      int* __restrict__ rinfo) {
  const int64_t units = n_idx * (d_c / 8);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units; u += stride) {
    const int64_t i = u / (d_c / 8);
    const int o = int(u - i * (d_c / 8)) * 8;
    const int64_t src = idx[i];
    if (o == 0) {
      int rows[KL];
#pragma unroll
      for (int q = 0; q < KL; ++q) rows[q] = -1;
      int cnt = 0, pos = -1;
      if (src >= 0 && src < total_rows) {
        const int b = int(src / T), t = int(src % T);
        pos = t;
        auto store_row = [&](int p) {
          if constexpr (FP8) {
            bool is_ref;
            const int j = tab ? ~tab[p] : refs_before(sv, p, is_ref);
            return b * sv.nref + min(max(j, 0), sv.nref - 1);   // records from rkv_encode: in range
          } else {
            return b * T + p;
          }
        };
        if (ref_idx[src * k] < 0) {                      // a reference: its own stored row
          rows[0] = store_row(t);
          cnt = 1;
        } else {
#pragma unroll
          for (int q = 0; q < KL; ++q) {
            const int p = q < k ? ref_idx[src * k + q] : -1;
            if (p >= 0) { rows[q] = store_row(p); ++cnt; }
          }
        }
      }
      int* ri = rinfo + i * (KL + 4);
#pragma unroll
      for (int q = 0; q < KL; ++q) ri[q] = rows[q];
      ri[KL] = __float_as_int(1.0f / float(max(cnt, 1)));
      ri[KL + 1] = pos;
    }
    // a reference token's ref_idx row is all -1 (every other token has at
    // least one reference: position 0 always is one)
    const bool live = src >= 0 && src < total_rows && ref_idx[src * k] >= 0;
    const int64_t sr = live ? src : 0;
    float zv[8];
    read_record8<BITS>(codes, scale, zmin, sr, o, d_c, g, zv);
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = live ? zv[e] : 0.0f;
      w[e] = sizeof(E) == 2 ? bf16_hi_lo(v) : __float_as_uint(v);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(zt + i * d_c + o);
    if constexpr (sizeof(E) == 2) {
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[e] = (w[2 * e] & 0xFFFFu) | (w[2 * e + 1] << 16);
        lv[e] = (w[2 * e] >> 16) | (w[2 * e + 1] & 0xFFFF0000u);
      }
      dst[0] = u32x4{hv[0], hv[1], hv[2], hv[3]};
      dst[1] = u32x4{lv[0], lv[1], lv[2], lv[3]};
    } else {
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
  }
}

// One workgroup: BM selected tokens x BN columns of KV^.  D divides BN, so a
// tile holds whole heads and every rotation partner (d +- D/2) is in it.
// The rows of the stored references whose mean it adds come from the prep
// kernel's table (FP8: rows of the E4M3 store).
// theta^(-2i/D) / (2 pi), the rotation rate of each of the D/2 <= 64 pairs
// of a head in revolutions per position, computed in fp64 on the host once
// per call (a kernel argument)
struct RateTable {
  double r[64];
};

template <typename E, typename CF>
constexpr int restore_main_lds() {
  if constexpr (sizeof(E) == 2)
    return DmaTileHL<CF::BM, CF::BN, CF::SB, CF::NS, CF::WGM, CF::WGN>::kLds;
  else
    return mainloop_lds<E, CF::BM, CF::BN, CF::SB, CF::NS, CF::WGM, CF::WGN>();
}

template <typename E, typename CF, int KL>
constexpr int restore_lds() {
  constexpr int LD = kEpiLd(CF::BN), HALF = CF::BM / 2;
  constexpr int kMain = restore_main_lds<E, CF>();
  constexpr int kStaged = kMain > HALF * LD * 4 ? kMain : HALF * LD * 4;
  return kStaged + CF::BM * (KL + 2) * 4 + 64 * 8;
}

// The tile at rows m0 .., columns n0 .. of KV^ (lds: restore_lds<E, CF, KL>()
// bytes, 1024-byte aligned).
// Eight consecutive stored values of a kv row (FP8 e4m3 references, bf16 or
// fp32), loaded as raw words and decoded to float separately, so that loads
// of several rows can be in flight before the first is used.
template <typename E, bool FP8> struct KvRaw {
  static constexpr int kBytes = FP8 ? 8 : 8 * int(sizeof(E));
  uint32_t w[kBytes / 4];
  __device__ __forceinline__ void load(const char* src) {
    if constexpr (kBytes == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(src);
      w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
      for (int h = 0; h < kBytes / 16; ++h) {
        const u32x4 x = reinterpret_cast<const u32x4*>(src)[h];
        w[4 * h] = x[0]; w[4 * h + 1] = x[1]; w[4 * h + 2] = x[2]; w[4 * h + 3] = x[3];
      }
    }
  }
  __device__ __forceinline__ void decode(float* v) const {
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = fp8_e4m3_to_f32((w[0] >> (8 * e)) & 0xFFu);
        v[4 + e] = fp8_e4m3_to_f32((w[1] >> (8 * e)) & 0xFFu);
      }
    } else if constexpr (sizeof(E) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(w[e]);
    }
  }
};

template <typename E, typename CF, int KL, bool FP8>
__device__ __forceinline__ void restore_tile(
    char* lds, int m0, int n0,
    const char* __restrict__ zt, const char* __restrict__ wdp, int K, int n_idx,
    const int* __restrict__ rinfo, const char* __restrict__ kv, int C, int ND, int D,
    float theta, const RateTable& rt, void* __restrict__ out, int out_bf16) {
  static_assert(CF::BN % 128 == 0, "a column tile holds whole heads (D divides 128)");
  constexpr int BM = CF::BM, BN = CF::BN, WGM = CF::WGM, WGN = CF::WGN, NT = CF::kThreads;
  static_assert(WGM == 2, "the epilogue stages one wave-row (half the tile) at a time");
  constexpr int LD = kEpiLd(BN);
  constexpr int HALF = BM / 2;
  constexpr int kMain = restore_main_lds<E, CF>();
  constexpr int kStaged = kMain > HALF * LD * 4 ? kMain : HALF * LD * 4;
  int* rows_lds = reinterpret_cast<int*>(lds + kStaged);            // [BM][KL] kv rows, -1 none
  float* inv_lds = reinterpret_cast<float*>(lds + kStaged + BM * KL * 4);  // [BM] 1 / count
  int* pos_lds = reinterpret_cast<int*>(lds + kStaged + BM * (KL + 1) * 4);  // [BM] t, -1 invalid
  double* rate = reinterpret_cast<double*>(lds + kStaged + BM * (KL + 2) * 4);  // [D/2] rates, revolutions
  const int tid = threadIdx.x;
  // The row's entry of the prep kernel's table: loaded before the main loop
  // (its latency passes under the first stages' copies), written to LDS
  // after it, where the epilogue's first barrier publishes it.  Rows past
  // n_idx repeat the last row; their results are not stored.
  static_assert(BM <= NT, "one row per thread");
  constexpr int kRI = (KL + 4) / 4;
  int4 ri[kRI];
  if (tid < BM) {
    const int4* src = reinterpret_cast<const int4*>(rinfo + size_t(min(m0 + tid, n_idx - 1)) * (KL + 4));
#pragma unroll
    for (int h = 0; h < kRI; ++h) ri[h] = src[h];
  }
  if (theta > 0.0f)
    for (int i = tid; i < D / 2; i += NT) rate[i] = rt.r[i];
  // K latents: a z~ row carries 4 bytes each (bf16 hi and lo, or fp32), a
  // packed W_d row one element each
  const size_t rowa = size_t(K) * 4, rowb = size_t(K) * sizeof(E);
  auto rowA = [&](int r) { return zt + size_t(min(m0 + r, n_idx - 1)) * rowa; };
  auto rowB = [&](int r) { return wdp + size_t(min(n0 + r, C - 1)) * rowb; };
  f32x16 acc[BM / WGM / 32][BN / WGN / 32];
  if constexpr (sizeof(E) == 2)
    tile_product_hl<BM, BN, CF::SB, CF::NS, WGM, WGN>(rowA, rowB, K, lds, acc);
  else
    tile_product<E, BM, BN, CF::SB, CF::NS, WGM, WGN>(rowA, rowB, int(rowb), lds, acc);
  if (tid < BM) {
    const int* v = reinterpret_cast<const int*>(ri);
#pragma unroll
    for (int q = 0; q < KL; ++q) rows_lds[tid * KL + q] = v[q];
    inv_lds[tid] = __int_as_float(v[KL]);
    pos_lds[tid] = v[KL + 1];
  }

  float* tile = reinterpret_cast<float*>(lds);
  constexpr int kV = BN / 8;                             // 8-column vectors per row
  const size_t kvrow = size_t(C) * (FP8 ? 1 : sizeof(E));
  constexpr int kUnits = HALF * kV;                      // 8-column units per half tile
  static_assert(kUnits % NT == 0, "every thread takes the same number of units");
  // units whose row loads are in flight together: at most 16 loads and 256
  // bytes per thread, 8 loads for eight FP8 rows a unit (whose e4m3 decode
  // would spill registers in the 8-wave tile)
  constexpr int kLoads = (FP8 && KL == 8) ? 8 : 16;
  constexpr int kB1 = 256 / (KL * KvRaw<E, FP8>::kBytes);
  constexpr int kB0 = kLoads / KL < kB1 ? kLoads / KL : kB1;
  constexpr int kB = kB0 < kUnits / NT ? kB0 : kUnits / NT;
  static_assert(kB >= 1 && (kUnits / NT) % kB == 0, "whole batches of units");
  for (int half = 0; half < 2; ++half) {
    acc_to_lds<BM, BN, WGM, WGN>(acc, tile, LD, half);
    __syncthreads();
    // a. + mean of the stored reference rows (NaN for an invalid index).
    // The row loads of kB units are issued before any is summed, so their
    // L2 round trips overlap; each unit's sum keeps the order q = 0..KL-1.
    // Columns past C load column 0 and store nothing.
    for (int u0 = 0; u0 < kUnits; u0 += kB * NT) {
      KvRaw<E, FP8> raw[kB][KL];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int u = u0 + j * NT + tid, rt = half * HALF + u / kV, col = n0 + (u % kV) * 8;
        const size_t off = size_t(col < C ? col : 0) * (FP8 ? 1 : sizeof(E));
#pragma unroll
        for (int q = 0; q < KL; ++q)
          raw[j][q].load(kv + size_t(max(rows_lds[rt * KL + q], 0)) * kvrow + off);
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int u = u0 + j * NT + tid, rl = u / kV, cv = (u % kV) * 8, rt = half * HALF + rl;
        if (n0 + cv >= C) continue;
        float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < KL; ++q) {
          float v[8];
          raw[j][q].decode(v);
          const bool ok = rows_lds[rt * KL + q] >= 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) m[e] += ok ? v[e] : 0.0f;
        }
        const float inv = inv_lds[rt];
        const bool bad = pos_lds[rt] < 0;
        float* tr = tile + rl * LD + cv;
#pragma unroll
        for (int e = 0; e < 8; ++e) tr[e] = bad ? __builtin_nanf("") : tr[e] + m[e] * inv;
      }
    }
    __syncthreads();
    // b. rotate K at the token's position, write the row
    for (int u = tid; u < HALF * kV; u += NT) {
      const int rl = u / kV, cv = (u % kV) * 8, rt = half * HALF + rl, col = n0 + cv;
      const int i = m0 + rt;
      if (col >= C || i >= n_idx) continue;
      float y[8];
      const float* tr = tile + rl * LD + cv;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = tr[e];
      const int pos = pos_lds[rt];
      if (theta > 0.0f && col < ND && pos >= 0) {
        const int d0 = col % D;                          // 8 columns in one half of a head
        const bool first = d0 < D / 2;
        const float* pr = tr + (first ? D / 2 : -(D / 2));
        const int i0 = first ? d0 : d0 - D / 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // angle pos * rate in revolutions, reduced to [-1/2, 1/2] in fp64,
          // then the hardware sine and cosine of revolutions
          const double a = double(pos) * rate[i0 + e];
          const float ar = float(a - rint(a));
          const float sn = __builtin_amdgcn_sinf(ar), cs = __builtin_amdgcn_cosf(ar);
          y[e] = first ? tr[e] * cs - pr[e] * sn : tr[e] * cs + pr[e] * sn;
        }
      }
      if (out_bf16) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = uint32_t(f32_to_bf16_rne(y[2 * e])) | (uint32_t(f32_to_bf16_rne(y[2 * e + 1])) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + size_t(i) * C + col) =
            u32x4{w[0], w[1], w[2], w[3]};
      } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + size_t(i) * C + col);
        o[0] = make_float4(y[0], y[1], y[2], y[3]);
        o[1] = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
    __syncthreads();
  }
}

// One launch of the restore: workgroups below n_wide take CF tiles over the
// rows [0, rows_wide) (whole rounds of the chip, or every row), the rest
// take CT tiles (the same wave count) over the rows [rows_wide, n_idx), so
// the part of the call that does not fill a round of CF tiles runs in
// smaller ones.  rows_wide is a multiple of CF::BM or n_idx; n_wide = 0,
// rows_wide = 0 gives a launch of CT tiles alone.
template <typename E, typename CF, typename CT, int KL, bool FP8>
__global__ __launch_bounds__(CF::kThreads, CF::kMinWaves) void k_restore(
    int n_wide, int rows_wide,
    const char* __restrict__ zt, const char* __restrict__ wdp, int K, int n_idx,
    const int* __restrict__ rinfo, const char* __restrict__ kv, int C, int ND, int D,
    float theta, RateTable rt, void* __restrict__ out, int out_bf16) {
  static_assert(CF::kThreads == CT::kThreads, "one block size");
  constexpr int kW = restore_lds<E, CF, KL>(), kT = restore_lds<E, CT, KL>();
  __shared__ __attribute__((aligned(1024))) char lds[kW > kT ? kW : kT];
  const int w = int(blockIdx.x);
  if (w < n_wide) {
    const int tm = (rows_wide + CF::BM - 1) / CF::BM;   // row tile fastest
    restore_tile<E, CF, KL, FP8>(lds, (w % tm) * CF::BM, (w / tm) * CF::BN, zt, wdp, K, n_idx,
                                 rinfo, kv, C, ND, D, theta, rt, out, out_bf16);
  } else {
    const int tm = (n_idx - rows_wide + CT::BM - 1) / CT::BM;
    const int u = w - n_wide;
    restore_tile<E, CT, KL, FP8>(lds, rows_wide + (u % tm) * CT::BM, (u / tm) * CT::BN, zt, wdp,
                                 K, n_idx, rinfo, kv, C, ND, D, theta, rt, out, out_bf16);
  }
}

// ------------------------------------------------------------------ gather-dequantise
template <int BITS, bool BF16>
__global__ __launch_bounds__(256) void k_gather(const uint8_t* __restrict__ codes,
                                                const uint16_t* __restrict__ scale,
                                                const uint16_t* __restrict__ zmin,
                                                const int32_t* __restrict__ idx, int64_t n_idx,
                                                int64_t total_rows, int d_c, int g,
                                                void* __restrict__ out) {
  const int64_t units = n_idx * (d_c / 8);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units; u += stride) {
    const int64_t f = u * 8;
    const int64_t i = f / d_c;
    const int o = int(f - i * d_c);
    const int64_t src = idx[i];
    float v[8];
    if (src < 0 || src >= total_rows) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
    } else {
      read_record8<BITS>(codes, scale, zmin, src, o, d_c, g, v);
    }
    if constexpr (BF16) {
      uint16_t* o16 = reinterpret_cast<uint16_t*>(out) + f;
      uint4 w;
      w.x = uint32_t(f32_to_bf16_rne(v[0])) | (uint32_t(f32_to_bf16_rne(v[1])) << 16);
      w.y = uint32_t(f32_to_bf16_rne(v[2])) | (uint32_t(f32_to_bf16_rne(v[3])) << 16);
      w.z = uint32_t(f32_to_bf16_rne(v[4])) | (uint32_t(f32_to_bf16_rne(v[5])) << 16);
      w.w = uint32_t(f32_to_bf16_rne(v[6])) | (uint32_t(f32_to_bf16_rne(v[7])) << 16);
      *reinterpret_cast<uint4*>(o16) = w;
    } else {
      float* o32 = reinterpret_cast<float*>(out) + f;
      *reinterpret_cast<float4*>(o32) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(o32 + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// P = R [W1 | W2] for the references a bf16 cache holds, rows in place: row
// m = b nref + j of R is kv row b T + p_j ([RKV] §2.2 mean eq.: the
// projections whose mean the append's mean branch takes); the encode's
// projection tiles on the same packed weights.
template <typename CF>
__global__ __launch_bounds__(CF::kThreads, 1) void k_ref_proj_rows(const char* __restrict__ kv,
                                                                   SchedView sv, int T, int C,
                                                                   int B,
                                                                   const char* __restrict__ wp,
                                                                   float* __restrict__ proj,
                                                                   int N, int tiles_m) {
  constexpr int kL = mainloop_lds<uint16_t, CF::BM, CF::BN, CF::SB, CF::NS, CF::WGM, CF::WGN>();
  __shared__ __attribute__((aligned(1024))) char lds[kL];
  const size_t rowb = size_t(C) * sizeof(uint16_t);
  const int nref = sv.nref;
  auto rowof = [&](int m) {
    return kv + (size_t(m / nref) * T + size_t(ref_position(sv, m % nref))) * rowb;
  };
  ref_proj_tile_rows<uint16_t, CF, true>(rowof, wp, proj, C, B * nref, N, tiles_m,
                                         int(blockIdx.x), lds);
}

int grid_for(int64_t work_items, int per_block) {
  const int64_t g = (work_items + per_block - 1) / per_block;
  return int(std::min<int64_t>(std::max<int64_t>(g, 1), 256 * 64));
}

}  // namespace

// ==================================================================== host
const Schedule& schedule_for(int T, int s0, double alpha, int n_sink) {
  thread_local Schedule last;
  if (last.T == T && last.s0 == s0 && last.alpha == alpha && last.n_sink == n_sink) return last;
  Schedule sc;
  sc.T = T; sc.s0 = s0; sc.alpha = alpha; sc.n_sink = n_sink;
  for (int t = 0; t < std::min(n_sink, T); ++t) sc.rpos.push_back(t);
  // p_{m+1} = p_m + s0 + floor(alpha * (p_m - n_sink)) ([RKV] §2.6), in
  // 64-bit integers and the floor of the double product
  for (long long p = n_sink; p < T;) {
    sc.rpos.push_back(int(p));
    p += s0 + (long long)std::floor(alpha * double(p - n_sink));
  }
  sc.nrp.reserve(size_t(T) - sc.rpos.size());
  size_t j = 0;
  for (int t = 0; t < T; ++t) {
    if (j < sc.rpos.size() && sc.rpos[j] == t) ++j;
    else sc.nrp.push_back(t);
  }
  last = std::move(sc);
  return last;
}

template <typename CF>
static int dist_items(const Shape& sh, int n_tt, int serp);

// How the distance launch deals token tiles to the XCDs: in turn (x, x + 8,
// ...), or alternating direction every row of 8 (serpentine), which evens
// the XCDs' item counts.  Measured in one process, per step: serpentine
// 0.4387 against 0.4459 ms at qwen7b_like_B2_T32k and 0.9692 against
// 0.9729 ms at multimodal_int2_B4_T16k, but 0.5436 against 0.5376 ms at
// llama8b_T32k (llama8b_T8k tied); so several sequences take it.
// RKV_DIST_DEAL=turn or =serp in the environment (read at every launch)
// forces either; both give the same bits.
static bool dist_serpentine(const Shape& sh) {
  const char* force = std::getenv("RKV_DIST_DEAL");
  if (force && !std::strcmp(force, "turn")) return false;
  if (force && !std::strcmp(force, "serp")) return true;
  return sh.B > 1;
}

// The distance launch's tiling for bf16 runs (fp32 runs: 0): narrow tiles
// (1) where the wide ones would give the chip fewer than two rounds of
// items, or where K = C <= 1024 makes the list scan (which a second
// workgroup per CU overlaps with matrix-core work) weigh most, on 128-
// reference chunks (2) in the first case.  Measured in one process, per
// step: llama8b_T8k 0.184 ms wide, 0.175 narrow, 0.137 narrow on 128-
// reference chunks; qwen7b_like_B2_T32k (C = 1024) 0.469 wide, 0.461 narrow
// (128-reference chunks tied, with a longer merge); llama8b_T32k wide
// (narrow 1.4% and 128-reference chunks 4% slower).  RKV_DIST_TILE=wide,
// =narrow or =short in the environment (read at every call) forces one; all
// give the same bits (the chunks only group the candidates of each token's
// lists, which the merge orders by (d, j)).
static int choose_dist_tiling(const Shape& sh) {
  if (!sh.bf16 || sh.nr == 0) return 0;
  const char* force = std::getenv("RKV_DIST_TILE");
  if (force && !std::strcmp(force, "wide")) return 0;
  if (force && !std::strcmp(force, "narrow")) return 1;
  if (force && !std::strcmp(force, "short")) return 2;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  using W = DistCfg<uint16_t>;
  if (dist_items<W>(sh, cdiv(sh.nr, W::BN), dist_serpentine(sh) ? 1 : 0) < 2 * cus) return 2;
  return sh.C <= 1024 ? 1 : 0;
}

Shape make_shape(int B, int T, int N, int D, int d_ff, int d_c, int k, int g, int b, int s,
                 bool bf16, double alpha, int n_sink, bool ref_fp8) {
  Shape sh{};
  sh.B = B; sh.T = T; sh.C = 2 * N * D; sh.d_ff = d_ff; sh.d_c = d_c; sh.k = k;
  sh.g = g; sh.b = b; sh.s = s; sh.bf16 = bf16;
  sh.alpha = alpha; sh.n_sink = n_sink; sh.ref_fp8 = ref_fp8;
  sh.esize = bf16 ? 2 : 4;
  sh.sched = &schedule_for(T, s, alpha, n_sink);
  sh.nref = int(sh.sched->rpos.size());
  sh.nr = T - sh.nref;
  sh.kl = k <= 4 ? 4 : 8;
  sh.dist_tiling = choose_dist_tiling(sh);
  sh.dist_bm = !bf16 ? DistCfg<float>::BM
             : sh.dist_tiling == 2 ? DistCfgShort::BM
             : sh.dist_tiling == 1 ? DistCfgNarrow::BM : DistCfg<uint16_t>::BM;
  sh.n_chunks = cdiv(sh.nref, sh.dist_bm);
  sh.k3 = d_ff;
  sh.kdh = bf16 ? 2 * d_ff : d_ff;
  return sh;
}

Workspace plan_workspace(const Shape& sh) {
  Workspace L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.wp = take(size_t(2) * sh.d_ff * sh.C * sh.esize);
  L.w3p = take(size_t(sh.d_c) * sh.k3 * sh.esize);
  L.ysq = take(size_t(sh.B) * sh.nref * 4);
  L.refs = take((size_t(sh.B) * sh.nref + 1) * sh.C * sh.esize);   // + the zero row
  L.proj = take(size_t(sh.B) * sh.nref * 2 * sh.d_ff * 4);
  L.part = take(size_t(sh.B) * cdiv(sh.nref, kMinChunk) * sh.nr * sh.kl * 8);
  L.dh = take(size_t(sh.B) * sh.nr * sh.kdh * sh.esize);
  L.rpos = take(size_t(sh.nref) * 4);
  L.nrp = take(size_t(sh.nr) * 4);
  L.tab = take(size_t(sh.T) * 4);
  L.selj = take(size_t(sh.B) * sh.nr * sh.kl * 4);
  L.total = off;
  return L;
}


hipError_t launch_store_refs(const Shape& sh, const void* kv, uint8_t* store, hipStream_t st) {
  const SchedView fixed{nullptr, sh.nref, sh.s, sh.n_sink};
  auto go = [&](const PosChunk& c, int use_chunk, int rows) {
    const int grid = cdiv(long(sh.B) * rows, 4);
    if (sh.bf16)
      k_ref_store<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(kv), sh.B, sh.T,
                                                  sh.C, fixed, c, use_chunk, sh.nref, store);
    else
      k_ref_store<float><<<grid, 256, 0, st>>>(static_cast<const float*>(kv), sh.B, sh.T, sh.C,
                                               fixed, c, use_chunk, sh.nref, store);
  };
  if (sh.alpha == 0.0) {
    PosChunk none;
    none.first = 0;
    none.count = 0;
    go(none, 0, sh.nref);
    return hipGetLastError();
  }
  // positions of a dynamic schedule ride in the kernel arguments, 960 at a time
  for (int first = 0; first < sh.nref; first += kPosChunk) {
    PosChunk c;
    c.first = first;
    c.count = std::min(kPosChunk, sh.nref - first);
    for (int i = 0; i < c.count; ++i) c.pos[i] = sh.sched->rpos[size_t(first) + i];
    go(c, 1, c.count);
  }
  return hipGetLastError();
}

hipError_t launch_ref_positions(const Shape& sh, int* rpos, hipStream_t st) {
  for (int first = 0; first < sh.nref; first += kPosChunk) {
    PosChunk c;
    c.first = first;
    c.count = std::min(kPosChunk, sh.nref - first);
    for (int i = 0; i < c.count; ++i) c.pos[i] = sh.sched->rpos[size_t(first) + i];
    k_sched_chunk<<<1, 256, 0, st>>>(rpos, c);
  }
  return hipGetLastError();
}

hipError_t launch_schedule(const Shape& sh, char* ws, const Workspace& L, hipStream_t st) {
  auto* rpos = reinterpret_cast<int*>(ws + L.rpos);
  auto* tab = reinterpret_cast<int*>(ws + L.tab);
  auto* nrp = reinterpret_cast<int*>(ws + L.nrp);
  if (sh.alpha == 0.0) {                                  // nref <= T: one thread per token
    k_sched_fixed<<<cdiv(sh.T, 256), 256, 0, st>>>(rpos, sh.nref, sh.T, sh.s, sh.n_sink, tab, nrp);
    return hipGetLastError();
  }
  const hipError_t e = launch_ref_positions(sh, rpos, st);
  if (e != hipSuccess) return e;
  k_sched_tables<<<cdiv(sh.T, 256), 256, 0, st>>>(rpos, sh.nref, sh.T, tab, nrp);
  return hipGetLastError();
}

hipError_t launch_setup(const Shape& sh, const void* w1, const void* w2, const void* w3,
                        const void* kv, char* ws, const Workspace& L, int32_t* ref_idx,
                        uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z,
                        hipStream_t st) {
  auto* rpos = reinterpret_cast<int*>(ws + L.rpos);
  const bool dynamic = sh.alpha != 0.0;
  if (dynamic) {                                         // positions first (kernel arguments)
    const hipError_t e = launch_ref_positions(sh, rpos, st);
    if (e != hipSuccess) return e;
  }
  PackJobs J{};
  int n_pack = 0;
  if (w1) {
    auto tiles = [](int n) { return (n + 63) / 64; };
    J.j[0] = {w1, ws + L.wp, sh.C, sh.d_ff, sh.C, 1, tiles(sh.d_ff), 0};
    J.j[1] = {w2, ws + L.wp, sh.C, sh.d_ff, sh.C, 2, tiles(sh.d_ff), 0};
    J.j[2] = {w3, ws + L.w3p, sh.d_ff, sh.d_c, sh.k3, 0, tiles(sh.d_c), 0};
    for (auto& j : J.j) {
      j.first = n_pack;
      n_pack += tiles(j.rows) * j.tiles_c;
    }
  } else {
    J.j[1].first = J.j[2].first = 0;
  }
  SchedArgs sa{dynamic ? rpos : nullptr, rpos, reinterpret_cast<int*>(ws + L.tab),
               reinterpret_cast<int*>(ws + L.nrp), sh.nref, sh.T, sh.s, sh.n_sink};
  const int n_tab = cdiv(sh.T, 256);
  RefArgs ra{};
  ra.kv = static_cast<const char*>(kv);
  ra.refs = ws + L.refs;
  ra.ysq = reinterpret_cast<float*>(ws + L.ysq);
  ra.ref_idx = ref_idx;
  ra.codes = codes;
  ra.scale = scale;
  ra.zmin = zmin;
  ra.z = z;
  ra.sv = SchedView{dynamic ? rpos : nullptr, sh.nref, sh.s, sh.n_sink};
  ra.B = sh.B; ra.T = sh.T; ra.C = sh.C; ra.nref = sh.nref; ra.k = sh.k;
  ra.cb = sh.d_c * sh.b / 8;
  ra.ng = sh.b == kIdentityBits ? 0 : sh.d_c / sh.g;     // identity mode stores no group numbers
  ra.d_c = sh.d_c;
  ra.fp8 = sh.ref_fp8;
  const int n_ref = cdiv(long(sh.B) * sh.nref + 1, 4);   // + the zero row
  const int grid = n_pack + n_tab + n_ref;
  if (sh.bf16)
    k_setup<uint16_t><<<grid, 256, 0, st>>>(J, n_pack, sa, n_tab, ra);
  else
    k_setup<float><<<grid, 256, 0, st>>>(J, n_pack, sa, n_tab, ra);
  return hipGetLastError();
}

size_t ref_proj_pack_bytes(const Shape& sh) {
  return sh.bf16 && !sh.ref_fp8 ? size_t(2) * sh.d_ff * sh.C * sh.esize : 0;
}

hipError_t launch_ref_proj_mfma(const Shape& sh, const void* kv, const void* w1, const void* w2,
                                const SchedView& sv, char* wp, float* proj, hipStream_t st) {
  // W1 | W2 packed as the encode packs them (rows of C, K-contiguous)
  auto tiles = [](int n) { return (n + 63) / 64; };
  PackJobs J{};
  J.j[0] = {w1, wp, sh.C, sh.d_ff, sh.C, 1, tiles(sh.d_ff), 0};
  J.j[1] = {w2, wp, sh.C, sh.d_ff, sh.C, 2, tiles(sh.d_ff), 0};
  int n_pack = 0;
  for (int i = 0; i < 2; ++i) {
    J.j[i].first = n_pack;
    n_pack += tiles(J.j[i].rows) * J.j[i].tiles_c;
  }
  J.j[2].first = n_pack;                                 // no third job
  k_pack_weights<uint16_t><<<n_pack, 256, 0, st>>>(J);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  using PF = DistCfg<uint16_t>::Proj;
  const int M = sh.B * sh.nref, N = 2 * sh.d_ff;
  const int tm = cdiv(M, PF::BM), tn = cdiv(N, PF::BN);
  k_ref_proj_rows<PF><<<tm * tn, PF::kThreads, 0, st>>>(static_cast<const char*>(kv), sv, sh.T,
                                                        sh.C, sh.B, wp, proj, N, tm);
  return hipGetLastError();
}

PackedLayout plan_packed(const Shape& sh) {
  PackedLayout P{};
  P.wp = 0;
  P.w3p = align256(size_t(2) * sh.d_ff * sh.C * sh.esize);
  P.total = P.w3p + align256(size_t(sh.d_c) * sh.k3 * sh.esize);
  return P;
}

hipError_t launch_pack_weights(const Shape& sh, const void* w1, const void* w2, const void* w3,
                               char* packed, hipStream_t st) {
  const PackedLayout P = plan_packed(sh);
  auto tiles = [](int n) { return (n + 63) / 64; };
  PackJobs J{};
  J.j[0] = {w1, packed + P.wp, sh.C, sh.d_ff, sh.C, 1, tiles(sh.d_ff), 0};
  J.j[1] = {w2, packed + P.wp, sh.C, sh.d_ff, sh.C, 2, tiles(sh.d_ff), 0};
  J.j[2] = {w3, packed + P.w3p, sh.d_ff, sh.d_c, sh.k3, 0, tiles(sh.d_c), 0};
  int n_pack = 0;
  for (auto& j : J.j) {
    j.first = n_pack;
    n_pack += tiles(j.rows) * j.tiles_c;
  }
  if (sh.bf16) k_pack_weights<uint16_t><<<n_pack, 256, 0, st>>>(J);
  else k_pack_weights<float><<<n_pack, 256, 0, st>>>(J);
  return hipGetLastError();
}

template <typename CF>
static int dist_items(const Shape& sh, int n_tt, int serp) {
  // per-XCD item counts (same enumeration as the kernel); grid = 8 x max
  constexpr int BM = CF::BM, BN = CF::BN;
  long per_xcd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int g = 0; g < sh.B * n_tt; ++g) {
    const int tt = g % n_tt;
    const int q = std::min(tt * BN + BN, sh.nr) - 1;
    const int np = sh.sched->nrp[q] - q;               // references before the tile's last token
    const int m = g >> 3, x = (serp && (m & 1)) ? 7 - (g & 7) : (g & 7);
    per_xcd[x] += (np + BM - 1) / BM;
  }
  return int(8 * *std::max_element(per_xcd, per_xcd + 8));
}

// Whether every tile of `rows` consecutive non-reference tokens (counted
// over all sequences when `flat`, within each sequence otherwise) has its kv
// rows, first to last, within 2^31 bytes: the reach of the buffer form of
// the main loop's DMA.  Rows between them are references; the host schedule
// gives the exact span.
// RKV_DMA_GLOBAL=1 in the environment (read at every launch) selects the
// global form everywhere; both forms compute the same bits.
static bool kv_tiles_fit_buffer(const Shape& sh, int rows, bool flat) {
  const char* force = std::getenv("RKV_DMA_GLOBAL");
  if (force && force[0] == '1') return false;
  const std::vector<int>& nrp = sh.sched->nrp;
  const int64_t nr = sh.nr, M = flat ? int64_t(sh.B) * nr : nr;
  auto pos = [&](int64_t q) { return (q / nr) * sh.T + nrp[size_t(q % nr)]; };
  int64_t span = 0;
  for (int64_t q0 = 0; q0 < M; q0 += rows)
    span = std::max(span, pos(std::min(q0 + rows - 1, M - 1)) - pos(q0));
  const int64_t rowb = int64_t(sh.C) * sh.esize;
  return (span + 1) * rowb < (int64_t(1) << 31);
}

hipError_t launch_dist(const Shape& sh, const void* kv, char* ws, const Workspace& L,
                       const char* wp, hipStream_t st) {
  if (sh.nr == 0) return hipGetLastError();
  const auto* p = static_cast<const char*>(kv);
  const auto* y = reinterpret_cast<const float*>(ws + L.ysq);
  auto* part = reinterpret_cast<float2*>(ws + L.part);
  const auto* nrp = reinterpret_cast<const int*>(ws + L.nrp);
  auto* proj = reinterpret_cast<float*>(ws + L.proj);
  const int pM = sh.B * sh.nref, pN = 2 * sh.d_ff;
  // the zero row after the reference block (written by the set-up), while
  // every reference row and it lie within one buffer resource's reach
  // (RKV_DIST_ZERO=0 in the environment, read at every launch, repeats a
  // reference row instead; the bits are the same)
  const size_t zoff = size_t(sh.B) * sh.nref * sh.C * sh.esize;
  const char* force_zero = std::getenv("RKV_DIST_ZERO");
  const bool use_zero = zoff + size_t(sh.C) * sh.esize < (size_t(1) << 31) &&
                        !(force_zero && !std::strcmp(force_zero, "0"));
  const char* zrow = use_zero ? ws + L.refs + zoff : nullptr;
  const int serp = dist_serpentine(sh) ? 1 : 0;
  auto go = [&](auto e, auto cf) {
    using E = decltype(e);
    using CF = decltype(cf);
    using PF = typename CF::Proj;
    const int n_tt = cdiv(sh.nr, CF::BN);
    const int n_dist = dist_items<CF>(sh, n_tt, serp);
    const int ptm = cdiv(pM, PF::BM);
    const int n_proj = wp != nullptr && pM > 0 ? ptm * cdiv(pN, PF::BN) : 0;
    const bool buf = sizeof(E) == 2 && kv_tiles_fit_buffer(sh, CF::BN, false);
#define RKV_DIST(KL, BUF)                                                                    \
    k_dist_topk<E, CF, KL, BUF><<<n_dist + n_proj, CF::kThreads, 0, st>>>(                   \
        p, ws + L.refs, y, part, sh.B, sh.T, sh.C, nrp, sh.nref, sh.nr, sh.n_chunks, n_tt,   \
        n_dist, wp, proj, pN, ptm, zrow, serp)
    if constexpr (sizeof(E) == 2) {
      if (sh.kl == 4) { if (buf) RKV_DIST(4, true); else RKV_DIST(4, false); }
      else { if (buf) RKV_DIST(8, true); else RKV_DIST(8, false); }
    } else {
      if (sh.kl == 4) RKV_DIST(4, false); else RKV_DIST(8, false);
    }
#undef RKV_DIST
  };
  if (!sh.bf16) go(float{}, DistCfg<float>{});
  else if (sh.dist_tiling == 2) go(uint16_t{}, DistCfgShort{});
  else if (sh.dist_tiling == 1) go(uint16_t{}, DistCfgNarrow{});
  else go(uint16_t{}, DistCfg<uint16_t>{});
  return hipGetLastError();
}

hipError_t launch_merge(const Shape& sh, int32_t* ref_idx, char* ws, const Workspace& L,
                        hipStream_t st) {
  const auto* part = reinterpret_cast<const float2*>(ws + L.part);
  const int nb = int(cdiv(long(sh.B) * sh.T * kMergeLanes, 256));
  const int chunk = sh.dist_bm;
  const auto* tab = reinterpret_cast<const int*>(ws + L.tab);
  const auto* rpos = reinterpret_cast<const int*>(ws + L.rpos);
#define RKV_MERGE(KL)                                                                        \
  k_topk_merge<KL><<<nb, 256, 0, st>>>(part, ref_idx, sh.B, sh.T, tab, rpos, sh.k, sh.nr,   \
                                      sh.n_chunks, chunk, reinterpret_cast<int*>(ws + L.selj))
  if (sh.kl == 4) RKV_MERGE(4); else RKV_MERGE(8);
#undef RKV_MERGE
  return hipGetLastError();
}

// k_swiglu's tile order.  With the row tile fastest, the kv rows are
// streamed once per column tile; the passes after the first find them in the
// 256 MB MALL while they fit there, and that order measured best at 128 MiB of
// kv rows (it also leaves them there for whatever reads kv next).  Once they
// outgrow it, every pass would fetch them from HBM again, and the column tile
// fastest order, which runs the column tiles of a token tile together, measured
// 6% faster at 256 MiB.  RKV_SWIGLU_ORDER=row or =col in the environment (read
// at every launch) forces one order; both compute the same bits.
static int swiglu_col_order(const Shape& sh) {
  const char* force = std::getenv("RKV_SWIGLU_ORDER");
  if (force && !std::strcmp(force, "row")) return 0;
  if (force && !std::strcmp(force, "col")) return 1;
  const double kv_bytes = double(sh.B) * sh.T * sh.C * (sh.bf16 ? 2.0 : 4.0);
  return kv_bytes > 192.0 * (1 << 20) ? 1 : 0;
}

// Whether k_swiglu writes delta_h non-temporally.  Where delta_h outgrows
// the caches, streaming it out keeps the kv rows and P columns that later
// tiles read again (measured per step in one process: multimodal_int2_B4_T16k,
// 252 MB of delta_h, 0.9636 -> 0.9509 ms; llama8b_T32k and
// qwen7b_like_B2_T32k, 126 MB, 1.5 us faster); where it fits, the W3 product
// finds it in the caches (llama8b_T8k, 31 MB: 3 us slower non-temporal).
// RKV_DH_NT=0 or =1 in the environment (read at every launch) forces either;
// the bits are the same.
static bool swiglu_nt(const Shape& sh) {
  const char* force = std::getenv("RKV_DH_NT");
  if (force && force[0] == '0') return false;
  if (force && force[0] == '1') return true;
  return double(sh.B) * sh.nr * sh.kdh * sh.esize > 64.0 * (1 << 20);
}

hipError_t launch_swiglu(const Shape& sh, const void* kv, char* ws,
                         const Workspace& L, const char* wp, hipStream_t st) {
  const int M = sh.B * sh.nr, N = 2 * sh.d_ff;
  if (M == 0) return hipGetLastError();
  const int col_order = swiglu_col_order(sh);
  const bool nt = swiglu_nt(sh);
  const auto* p = static_cast<const char*>(kv);
  const auto* proj = reinterpret_cast<const float*>(ws + L.proj);
  // P is addressed with 32-bit byte offsets (its size is checked on the host)
  const uint32_t pbytes = uint32_t(size_t(sh.B) * sh.nref * N * 4);
#define RKV_SW(E, KL, BUF, ST)                                                                  \
  k_swiglu<E, KL, BUF, ST><<<cdiv(N, SwCfg<E>::BN) * cdiv(M, SwCfg<E>::BM), SwCfg<E>::kThreads, \
                             0, st>>>(                                                          \
      p, wp, proj, pbytes, reinterpret_cast<const int*>(ws + L.selj), ws + L.dh, sh.T,          \
      sh.C, reinterpret_cast<const int*>(ws + L.nrp), sh.nref, sh.nr, sh.d_ff, M, col_order)
#define RKV_SW_NT(E, KL, BUF) \
  if (nt) RKV_SW(E, KL, BUF, true); else RKV_SW(E, KL, BUF, false);
  if (sh.bf16) {
    const bool buf = kv_tiles_fit_buffer(sh, SwCfg<uint16_t>::BM, true);
    if (sh.kl == 4) { if (buf) { RKV_SW_NT(uint16_t, 4, true) } else { RKV_SW_NT(uint16_t, 4, false) } }
    else { if (buf) { RKV_SW_NT(uint16_t, 8, true) } else { RKV_SW_NT(uint16_t, 8, false) } }
  } else {
    if (sh.kl == 4) RKV_SW(float, 4, false, false); else RKV_SW(float, 8, false, false);
  }
#undef RKV_SW_NT
#undef RKV_SW
  return hipGetLastError();
}

// The narrow bf16 W3 tiles where the wide ones would number fewer than half
// the CUs (llama8b_T8k: 60 wide tiles).  RKV_W3_TILE=wide or =narrow in the
// environment (read at every launch) forces one; the tile shape changes no
// output's accumulation order, so both give the same bits.
static bool w3_narrow(const Shape& sh) {
  if (!sh.bf16) return false;
  const char* force = std::getenv("RKV_W3_TILE");
  if (force && !std::strcmp(force, "wide")) return false;
  if (force && !std::strcmp(force, "narrow")) return true;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  using W = W3Cfg<uint16_t>;
  const long wide = long(cdiv(sh.d_c, W::BN)) * cdiv(long(sh.B) * sh.nr, W::BM);
  return 2 * wide < cus;
}

hipError_t launch_w3_quant(const Shape& sh, char* ws, const Workspace& L, const char* w3p,
                           uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z,
                           hipStream_t st) {
  const int M = sh.B * sh.nr, N = sh.d_c;
  if (M == 0) return hipGetLastError();
  const char* a = ws + L.dh;
  const char* w = w3p;
  auto go = [&](auto e, auto cf) {
    using E = decltype(e);
    using CF = decltype(cf);
    const int tm = cdiv(M, CF::BM);
#define RKV_W3(BITS, G8)                                                                      \
    k_w3_quant<E, CF, BITS, G8><<<cdiv(N, CF::BN) * tm, CF::kThreads, 0, st>>>(               \
        a, w, sh.k3, M, N, tm, sh.T, reinterpret_cast<const int*>(ws + L.nrp), sh.nr, codes,  \
        scale, zmin, z)
#define RKV_W3G(BITS)                         \
    switch (sh.g) {                           \
      case 8: RKV_W3(BITS, 1); break;         \
      case 16: RKV_W3(BITS, 2); break;        \
      case 32: RKV_W3(BITS, 4); break;        \
      default: RKV_W3(BITS, 8); break;        \
    }
    if (sh.b == 4) { RKV_W3G(4) } else if (sh.b == 2) { RKV_W3G(2) }
    else { RKV_W3(kIdentityBits, 1); }
#undef RKV_W3G
#undef RKV_W3
  };
  if (!sh.bf16) go(float{}, W3Cfg<float>{});
  else if (w3_narrow(sh)) go(uint16_t{}, W3CfgNarrow{});
  else go(uint16_t{}, W3Cfg<uint16_t>{});
  return hipGetLastError();
}

hipError_t launch_quantize(const float* z, int64_t rows, int d_c, int g, int b, uint8_t* codes,
                           uint16_t* scale, uint16_t* zmin, hipStream_t st) {
  if (rows == 0) return hipGetLastError();
  const int64_t units = rows * (d_c / 8);
  const int grid = grid_for(units, 256);
#define RKV_Q(BITS, G8) k_quantize<BITS, G8><<<grid, 256, 0, st>>>(z, rows, d_c, codes, scale, zmin)
#define RKV_QG(BITS)                        \
  switch (g) {                              \
    case 8: RKV_Q(BITS, 1); break;          \
    case 16: RKV_Q(BITS, 2); break;         \
    case 32: RKV_Q(BITS, 4); break;         \
    default: RKV_Q(BITS, 8); break;         \
  }
  if (b == 4) { RKV_QG(4) } else if (b == 2) { RKV_QG(2) } else { RKV_Q(kIdentityBits, 1); }
#undef RKV_QG
#undef RKV_Q
  return hipGetLastError();
}

hipError_t launch_gather(const uint8_t* codes, const uint16_t* scale, const uint16_t* zmin,
                         const int32_t* idx, int64_t n_idx, int64_t total_rows, int d_c, int g,
                         int b, void* out, bool out_bf16, hipStream_t st) {
  if (n_idx == 0) return hipGetLastError();
  const int64_t units = n_idx * (d_c / 8);
  const int grid = grid_for(units, 256);
#define RKV_G(BITS, BF) \
  k_gather<BITS, BF><<<grid, 256, 0, st>>>(codes, scale, zmin, idx, n_idx, total_rows, d_c, g, out)
  if (b == 4) { if (out_bf16) RKV_G(4, true); else RKV_G(4, false); }
  else if (b == 2) { if (out_bf16) RKV_G(2, true); else RKV_G(2, false); }
  else { if (out_bf16) RKV_G(kIdentityBits, true); else RKV_G(kIdentityBits, false); }
#undef RKV_G
  return hipGetLastError();
}

RestoreWorkspace plan_restore(const Shape& sh, int64_t n_idx) {
  RestoreWorkspace L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.kr = sh.d_c;
  L.wdp = take(size_t(sh.C) * L.kr * sh.esize);
  L.zt = take(size_t(n_idx) * sh.d_c * 4);
  L.rinfo = take(size_t(n_idx) * (sh.kl + 4) * 4);
  L.tables = sh.ref_fp8 && sh.alpha != 0.0;        // FP8 rows of a dynamic schedule: tab[p]
  if (L.tables) {
    L.rpos = take(size_t(sh.nref) * 4);
    L.nrp = take(size_t(sh.nr) * 4);
    L.tab = take(size_t(sh.T) * 4);
  }
  L.total = off;
  return L;
}

// The restore's tiling (bf16): narrow tiles where the wide ones would fill at
// most half the CUs.  Measured in one process at C = 2048 (calls of
// rkv_restore): 1,024 rows 72.5 -> 40.8 us, 4,096 rows 75.1 -> 49.4 us; at
// 9,830 rows (1.2 rounds of wide tiles) narrow tiles lost, 118 against 104
// us, as they did at 32,768 rows (312 against 265 us), on twice the operand
// traffic per flop.  RKV_RESTORE_TILE=narrow in the environment (read at
// every launch) forces them, any other value the 8-wave tiles
// (restore_wide_rows); every tiling gives the same bits.
static bool restore_narrow(const Shape& sh, int n_idx) {
  if (!sh.bf16) return false;
  const char* force = std::getenv("RKV_RESTORE_TILE");
  if (force && !std::strcmp(force, "narrow")) return true;
  if (force) return false;                             // a forced 8-wave split
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  using W = RsCfg<uint16_t>;
  const long wide = long(cdiv(n_idx, W::BM)) * cdiv(sh.C, W::BN);
  return 2 * wide <= cus;
}

// Rows of a bf16 restore that go to 256 x 256 tiles: the whole rounds of
// them (one tile per CU) when there is at least one and the rows after fit
// in one round of 128 x 256 tiles; else every row.  In one process at
// C = 2048, per call: 9,830 rows 102.8 -> 98.9 us (8,192 rows in one round
// of 256 wide tiles, then 104 half tiles), 12,000 rows 124.3 -> 111.1 us,
// 20,000 rows 176.7 -> 168.0 us; at 6,000 rows (no whole round) half tiles
// alone lost, 78.4 against 71.9 us.  RKV_RESTORE_TILE (read at every launch)
// forces the split: =wide every row in wide tiles, =tail none, =<rows> that
// many rows (rounded down to a multiple of 256).
static int restore_wide_rows(const Shape& sh, int n_idx) {
  constexpr int WBM = RsCfg<uint16_t>::BM;
  const char* force = std::getenv("RKV_RESTORE_TILE");
  if (force && !std::strcmp(force, "wide")) return n_idx;
  if (force && !std::strcmp(force, "tail")) return 0;
  if (force && force[0] >= '0' && force[0] <= '9')
    return std::min(std::atoi(force) / WBM * WBM, n_idx / WBM * WBM);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int per_round = std::max(1, cus / cdiv(sh.C, RsCfg<uint16_t>::BN)) * WBM;
  const int full = n_idx / per_round * per_round;
  const int tail_tiles = cdiv(n_idx - full, RsCfgTail::BM) * cdiv(sh.C, RsCfgTail::BN);
  return full > 0 && tail_tiles <= cus ? full : n_idx;
}

size_t packed_decoder_bytes(const Shape& sh) {
  return size_t(sh.C) * sh.d_c * sh.esize;
}

hipError_t launch_pack_decoder(const Shape& sh, const void* wd, char* wdp, hipStream_t st) {
  // W_d [d_c][C] -> [C][d_c] K-contiguous rows
  PackJobs J{};
  J.j[0] = {wd, wdp, sh.d_c, sh.C, sh.d_c, 0, (sh.C + 63) / 64, 0};
  const int tiles = (sh.d_c + 63) / 64 * J.j[0].tiles_c;
  J.j[1].first = tiles;
  J.j[2].first = tiles;
  if (sh.bf16) k_pack_weights<uint16_t><<<tiles, 256, 0, st>>>(J);
  else k_pack_weights<float><<<tiles, 256, 0, st>>>(J);
  return hipGetLastError();
}

hipError_t launch_restore(const Shape& sh, int N, int D, const uint8_t* codes,
                          const uint16_t* scale, const uint16_t* zmin, const int32_t* ref_idx,
                          const void* kv, const char* wdp, const int32_t* idx, int n_idx,
                          float theta, void* out, bool out_bf16, char* ws,
                          const RestoreWorkspace& L, hipStream_t st) {
  if (n_idx == 0) return hipGetLastError();
  const int64_t total = int64_t(sh.B) * sh.T;
  const SchedView sv{nullptr, sh.nref, sh.s, sh.n_sink};
  const int* tab = nullptr;
  if (L.tables) {
    Workspace T{};
    T.rpos = L.rpos; T.nrp = L.nrp; T.tab = L.tab;
    const hipError_t e = launch_schedule(sh, ws, T, st);
    if (e != hipSuccess) return e;
    tab = reinterpret_cast<const int*>(ws + L.tab);
  }
  const int grid = grid_for(int64_t(n_idx) * (sh.d_c / 8), 256);
  auto* zt = reinterpret_cast<uint32_t*>(ws + L.zt);
  auto* rinfo = reinterpret_cast<int*>(ws + L.rinfo);
  auto prep = [&](auto e, auto bits_c) {
    using E = decltype(e);
    constexpr int BITS = decltype(bits_c)::value;
#define RKV_RP(KL, F8)                                                                        \
    k_restore_prep<E, BITS, KL, F8><<<grid, 256, 0, st>>>(codes, scale, zmin, idx, n_idx, total, \
                                                          ref_idx, sh.k, sh.d_c, sh.g, zt, sh.T, \
                                                          sv, tab, rinfo)
    if (sh.ref_fp8) { if (sh.kl == 4) RKV_RP(4, true); else RKV_RP(8, true); }
    else { if (sh.kl == 4) RKV_RP(4, false); else RKV_RP(8, false); }
#undef RKV_RP
  };
  using B4 = std::integral_constant<int, 4>;
  using B2 = std::integral_constant<int, 2>;
  using BI = std::integral_constant<int, kIdentityBits>;
  if (sh.bf16) {
    if (sh.b == 4) prep(uint16_t{}, B4{}); else if (sh.b == 2) prep(uint16_t{}, B2{});
    else prep(uint16_t{}, BI{});
  } else {
    if (sh.b == 4) prep(float{}, B4{}); else if (sh.b == 2) prep(float{}, B2{});
    else prep(float{}, BI{});
  }
  const auto* kvp = static_cast<const char*>(kv);
  RateTable rt{};
  if (theta > 0.0f)
    for (int i = 0; i < D / 2; ++i)   // in revolutions per position
      rt.r[i] = std::pow(double(theta), -2.0 * i / double(D)) / 6.283185307179586;
  // n_wide CF tiles over rows [0, rows_wide), then CT tiles over the rest
  auto go = [&](auto e, auto cf, auto ct, int rows_wide) {
    using E = decltype(e);
    using CF = decltype(cf);
    using CT = decltype(ct);
    const int n_wide = cdiv(rows_wide, CF::BM) * cdiv(sh.C, CF::BN);
    const int grid = n_wide + cdiv(n_idx - rows_wide, CT::BM) * cdiv(sh.C, CT::BN);
#define RKV_RS(KL, F8)                                                                          \
    k_restore<E, CF, CT, KL, F8><<<grid, CF::kThreads, 0, st>>>(                              \
        n_wide, rows_wide, ws + L.zt, wdp, L.kr, n_idx, rinfo, kvp, sh.C, N * D, D,           \
        theta, rt, out, out_bf16 ? 1 : 0)
    if (sh.ref_fp8) { if (sh.kl == 4) RKV_RS(4, true); else RKV_RS(8, true); }
    else { if (sh.kl == 4) RKV_RS(4, false); else RKV_RS(8, false); }
#undef RKV_RS
  };
  if (!sh.bf16) go(float{}, RsCfg<float>{}, RsCfg<float>{}, 0);
  else if (restore_narrow(sh, n_idx)) go(uint16_t{}, RsCfgNarrow{}, RsCfgNarrow{}, 0);
  else go(uint16_t{}, RsCfg<uint16_t>{}, RsCfgTail{}, restore_wide_rows(sh, n_idx));
  return hipGetLastError();
}

}  // namespace rkv
