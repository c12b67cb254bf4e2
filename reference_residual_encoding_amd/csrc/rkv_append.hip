// Decode-time append of the ResidualKV cache ([RKV] §2.7, decode step 4):
// one new token per sequence is either stored as it is, when the schedule
// of [RKV] §2.6 makes its position a reference, or encoded against the
// references already in the cache ([RKV] §2.2-§2.4) and stored as a record.
//
// The work per call is a few vectors against the cache and the weights, so
// every kernel here is a streaming kernel on the vector ALUs, in fp32 from
// the stored values (no matrix cores: at one to a few dozen tokens the
// products are bound by reading the weights and the references once):
//   dist     one workgroup per 8 pool references of a sequence: squared L2
//            by direct differences, the workgroup's best KL as a list
//   sel_proj one workgroup per 16 features, slice of the C rows and 2 or 4
//            tokens: each merges its tokens' lists by (distance, position)
//            itself, then x W1, x W2, m W1, m W2 over its rows (the mean m of
//            the chosen references formed in fp32 at the rows it needs),
//            reduced in LDS to one partial sum per slice; the first feature
//            block writes ref_idx, and stores a reference token in the cache
//            with a zero record
//   w3       one workgroup per (token, 32 or 64 latent columns): the slices'
//            partial sums added in slice order, delta_h = Swish(x W1) (x W2)
//            - Swish(m W1) (m W2) ([RKV] §2.3), z = delta_h W3 (W3 is
//            linear, so f_c(kv) - f_c(m) = (h(kv) - h(m)) W3), then the group
//            quantiser of [RKV] §2.4 and the record
// With the references' projections P = R [W1 | W2] kept beside the cache
// (rkv_append_proj), two launches do the same: dist_xproj (the distance
// workgroups and, in the same grid, x [W1 | W2] in slices of the C rows)
// and sel_w3 (per token and column block: the selection, m [W1 | W2] as the
// mean of k_t rows of P, delta_h, W3 and the quantiser); ref_proj fills P
// on the vector ALUs where the matrix-core tiles do not apply.
#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_quant.h"

#include <cfloat>
#include <cstdlib>
#include <mutex>
#include <type_traits>

namespace rkv {

namespace {

constexpr int kAppCH = 8;          // pool references per distance workgroup (4 waves x 2)
constexpr int kNoRef = 0x7fffffff;  // list padding (sorts after every reference)

template <typename E>
__device__ __forceinline__ void load8(const E* p, float (&v)[8]) {
  if constexpr (sizeof(E) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Four consecutive weights loaded as raw words now and converted to float
// later, so the load can be requested ahead of its use.
template <typename E> struct RawW4;
template <> struct RawW4<uint16_t> {
  uint2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void decode(float (&v)[4]) const {
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  }
};
template <> struct RawW4<float> {
  float4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void decode(float (&v)[4]) const {
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
};

template <typename E>
__device__ __forceinline__ float load1(const E* p) {
  if constexpr (sizeof(E) == 2) return bf16_to_f32(*p);
  else return *p;
}

// Eight consecutive values loaded as raw words now and converted to float
// later, so that a batch of loads can be requested before any is used.
template <typename E> struct RawW8;
template <> struct RawW8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void decode(float (&v)[8]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
};
template <> struct RawW8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void decode(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename E> struct RawF8x8 {                   // 8 E4M3 bytes
  uint2 w;
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void decode(float (&v)[8]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = fp8_e4m3_to_f32((w.x >> (8 * e)) & 0xFFu);
      v[4 + e] = fp8_e4m3_to_f32((w.y >> (8 * e)) & 0xFFu);
    }
  }
};

// Stored reference j of sequence b: the row at its position in kv
// [B][T][C] (input precision), or row j of the FP8 store [B][nref][C].
template <typename E, bool FP8>
struct RefRows {
  const void* base;
  SchedView sv;
  int T, C;
  __device__ __forceinline__ size_t row(int b, int j) const {
    return FP8 ? size_t(b) * sv.nref + j : size_t(b) * T + ref_position(sv, j);
  }
  // 8 coordinates [o, o + 8) of stored row `r` (from row()), raw
  using Raw = std::conditional_t<FP8, RawF8x8<E>, RawW8<E>>;
  __device__ __forceinline__ void load_raw(size_t r, int o, Raw& w) const {
    if constexpr (FP8)
      w.load(static_cast<const uint8_t*>(base) + r * C + o);
    else
      w.load(static_cast<const E*>(base) + r * C + o);
  }
  // the same, converted
  __device__ __forceinline__ void load(size_t r, int o, float (&v)[8]) const {
    if constexpr (FP8) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + r * C + o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = fp8_e4m3_to_f32((w.x >> (8 * e)) & 0xFFu);
        v[4 + e] = fp8_e4m3_to_f32((w.y >> (8 * e)) & 0xFFu);
      }
    } else {
      load8(static_cast<const E*>(base) + r * C + o, v);
    }
  }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// State of a new token at position t: -1 nothing to encode (invalid
// position or a reference), else the size of its pool.
__device__ __forceinline__ int pool_at(const SchedView& v, int t, int T) {
  if (t < 0 || t >= T) return -1;
  bool is_ref;
  const int n = refs_before(v, t, is_ref);
  return is_ref ? -1 : n;
}

// ---------------------------------------------------------------- distance
// Workgroup (b, c): pool references j in [8c, 8c + 8) of sequence b, two
// per wave with both rows' loads in flight; d = sum (x - y)^2 in fp32.  The
// rows are requested before the pool is known (j clamped into the
// references), together with the position's load.  The workgroup's list is
// then ranked in parallel: each of 8 lanes counts the candidates that order
// before its own by (d, j), and candidates that no list slot would take
// (past the pool, or d not <= FLT_MAX) leave their slots to padding.
template <typename E, int KL, bool FP8, int U>
__device__ __forceinline__ void dist_block(const void* __restrict__ kv,
                                           const E* __restrict__ kv_new,
                                           const int32_t* __restrict__ pos, SchedView sv, int T,
                                           int C, int n_lists, float2* __restrict__ part,
                                           int blk) {
  const RefRows<E, FP8> refs{kv, sv, T, C};
  if (sv.nref <= 0) return;                              // no references: no lists
  const int b = blk / n_lists, c = blk % n_lists;
  const int j0 = c * kAppCH;
  __shared__ float dl[kAppCH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ja = j0 + 2 * wave, jb = ja + 1;
  const E* x = kv_new + size_t(b) * C;
  const size_t ya = refs.row(b, min(ja, sv.nref - 1)), yb = refs.row(b, min(jb, sv.nref - 1));
  // the position through a vector load requested after the rows' addresses
  // are known: its wait then comes after the rows' (a scalar load would be
  // waited for with the kernel arguments the loop needs)
  asm volatile("" ::: "memory");
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  const int t = pos[b + zero];
  float sa = 0.0f, sb = 0.0f;
  // U x 512 coordinates at a time: all 3U loads of a lane requested before
  // any is used (coordinates past C read coordinate 0 and add nothing)
  for (int o0 = 0; o0 < C; o0 += U * 512) {
    RawW8<E> xr[U];
    typename RefRows<E, FP8>::Raw ar[U], br[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o = o0 + u * 512 + lane * 8;
      const int oc = o < C ? o : 0;
      xr[u].load(x + oc);
      refs.load_raw(ya, oc, ar[u]);
      refs.load_raw(yb, oc, br[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = o0 + u * 512 + lane * 8 < C;
      float xv[8], av[8], bv[8];
      xr[u].decode(xv);
      ar[u].decode(av);
      br[u].decode(bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float da = in ? xv[e] - av[e] : 0.0f, db = in ? xv[e] - bv[e] : 0.0f;
        sa = fmaf(da, da, sa);
        sb = fmaf(db, db, sb);
      }
    }
  }
  asm volatile("" ::: "memory");                        // the row loads stay ahead of the exit
  const int pool = pool_at(sv, t, T);                    // uniform over the workgroup
  if (pool < 0 || j0 >= pool) return;
  sa = wave_sum(sa);
  sb = wave_sum(sb);
  if (lane == 0) {
    dl[2 * wave] = sa;
    dl[2 * wave + 1] = sb;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    static_assert(kAppCH <= 64 && KL <= kAppCH, "one lane per candidate and per slot");
    const int i = lane;
    const float di = dl[min(i, kAppCH - 1)];
    // a slot takes (d, j) when it orders before the padding (FLT_MAX, kNoRef)
    const bool ok = i < kAppCH && j0 + i < pool && di <= FLT_MAX;
    int rank = 0;
#pragma unroll
    for (int e = 0; e < kAppCH; ++e) {
      const float de = dl[e];
      const bool oe = j0 + e < pool && de <= FLT_MAX;
      rank += (oe && (de < di || (de == di && e < i))) ? 1 : 0;
    }
    const int n_ok = __popcll(__ballot(ok));
    float2* dst = part + size_t(blk) * KL;
    if (ok && rank < KL) dst[rank] = make_float2(di, __int_as_float(j0 + i));
    if (i >= n_ok && i < KL) dst[i] = make_float2(FLT_MAX, __int_as_float(kNoRef));
  }
}

template <typename E, int KL, bool FP8, int U>
__global__ __launch_bounds__(256) void k_app_dist(const void* __restrict__ kv,
                                                  const E* __restrict__ kv_new,
                                                  const int32_t* __restrict__ pos, SchedView sv,
                                                  int T, int C, int n_lists,
                                                  float2* __restrict__ part) {
  dist_block<E, KL, FP8, U>(kv, kv_new, pos, sv, T, C, n_lists, part, int(blockIdx.x));
}

// ---------------------------------------------------------------- select + projection
// One launch does both: every workgroup (16 features of RB appended tokens,
// one slice of rows) first chooses its tokens' references itself, from the
// distance lists (they are small and L2-resident), so no launch waits for a
// separate selection.  The workgroup of feature block 0 and slice 0 also
// writes the token's ref_idx, stores a reference token as it is (with a
// zero record) and sets act[b] = 1 when the token is to be encoded.
//
// Selection of sequence b's token by one wave: every lane merges the lists
// l, l + 64, ... of the ceil(pool/8) lists, then the lanes' lists are merged
// by a butterfly over the wave (each a merge of two sorted lists,
// merge_sorted_lex); by (distance, position), which orders every
// candidate uniquely, so the kept k_t = min(k, |pool|) ([RKV] §2.1) do not
// depend on the merge order.  Writes the chosen stored rows (ascending
// position) to sel[0..KL), and their reference indices to selj[0..KL) when
// selj is given, and returns k_t; -1 when the token is not encoded (no
// append this call, or a reference).  With `writer`, also writes
// ref_idx and act[b], and stores a reference token as it is.  `pre()` is
// called once, right after the first lists are requested (the caller's own
// loads then queue behind them, not in front).  b must be uniform over the
// wave.
template <typename E, int KL, bool FP8, typename Pre>
__device__ int select_token(void* kv, const E* kv_new, const int32_t* pos, SchedView sv, int T,
                            int C, int k, int rec_bytes, int n_groups, int d_c, int n_lists,
                            const float2* part, int32_t* ref_idx, uint8_t* codes, uint16_t* scale,
                            uint16_t* zmin, float* z, int* act, int b, bool writer, int* sel,
                            Pre pre, int* selj = nullptr) {
  const int lane = threadIdx.x & 63;
  const int t = pos[b];
  // The lists' addresses do not depend on the position: the first LU per
  // lane are requested together with it (l >= n_lists reads the last list;
  // only lists below the pool's count are merged, as padding otherwise).
  constexpr int LU = 4;
  float4 w[LU][KL / 2];
  auto request = [&](int l0) {
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      const int l = min(l0 + 64 * u, n_lists - 1);
      const float4* src = reinterpret_cast<const float4*>(part + (size_t(b) * n_lists + l) * KL);
#pragma unroll
      for (int e = 0; e < KL / 2; ++e) w[u][e] = src[e];
    }
  };
  request(lane);
  // the lists' loads, then pre()'s, then the rest: nothing moves across
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  pre();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (t < 0 || t >= T) {                                 // not appended this call
    if (writer && act && lane == 0) act[b] = 0;
    return -1;
  }
  const size_t row = size_t(b) * T + t;
  bool is_ref;
  const int pool = refs_before(sv, t, is_ref);
  const RefRows<E, FP8> refs{kv, sv, T, C};
  if (is_ref) {                                          // stored as it is ([RKV] §2.4)
    if (!writer) return -1;
    for (int o = lane * 8; o < C; o += 64 * 8) {
      if constexpr (FP8) {                               // its E4M3 bytes, row j = pool
        float v[8];
        load8(kv_new + size_t(b) * C + o, v);
        uint2 w;
        w.x = f32_to_fp8_e4m3(v[0]) | (f32_to_fp8_e4m3(v[1]) << 8) |
              (f32_to_fp8_e4m3(v[2]) << 16) | (f32_to_fp8_e4m3(v[3]) << 24);
        w.y = f32_to_fp8_e4m3(v[4]) | (f32_to_fp8_e4m3(v[5]) << 8) |
              (f32_to_fp8_e4m3(v[6]) << 16) | (f32_to_fp8_e4m3(v[7]) << 24);
        *reinterpret_cast<uint2*>(static_cast<uint8_t*>(kv) + refs.row(b, pool) * C + o) = w;
      } else if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<u32x4*>(static_cast<E*>(kv) + row * C + o) =
            *reinterpret_cast<const u32x4*>(kv_new + size_t(b) * C + o);
      } else {
        reinterpret_cast<float4*>(static_cast<E*>(kv) + row * C + o)[0] =
            reinterpret_cast<const float4*>(kv_new + size_t(b) * C + o)[0];
        reinterpret_cast<float4*>(static_cast<E*>(kv) + row * C + o)[1] =
            reinterpret_cast<const float4*>(kv_new + size_t(b) * C + o)[1];
      }
    }
    for (int i = lane; i < k; i += 64) ref_idx[row * k + i] = -1;
    for (int i = lane; i < rec_bytes; i += 64) codes[row * rec_bytes + i] = 0;
    for (int i = lane; i < n_groups; i += 64) {
      scale[row * n_groups + i] = 0;
      zmin[row * n_groups + i] = 0;
    }
    if (z)
      for (int i = lane; i < d_c; i += 64) z[row * d_c + i] = 0.0f;
    if (act && lane == 0) act[b] = 0;
    return -1;
  }
  const int nch = (pool + kAppCH - 1) / kAppCH;
  float bd[KL];
  int bi[KL];
#pragma unroll
  for (int e = 0; e < KL; ++e) { bd[e] = FLT_MAX; bi[e] = kNoRef; }
  auto merge = [&](int l0) {
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      // a list past the pool's enters as padding, which no slot takes (the
      // loads are used either way, so none is moved under a branch); each
      // list is in ascending (d, j) order
      const bool in = l0 + 64 * u < nch;
      float ld[KL];
      int li[KL];
#pragma unroll
      for (int e = 0; e < KL / 2; ++e) {
        ld[2 * e] = in ? w[u][e].x : FLT_MAX;
        li[2 * e] = in ? __float_as_int(w[u][e].y) : kNoRef;
        ld[2 * e + 1] = in ? w[u][e].z : FLT_MAX;
        li[2 * e + 1] = in ? __float_as_int(w[u][e].w) : kNoRef;
      }
      merge_sorted_lex(bd, bi, ld, li);
    }
  };
  merge(lane);
  for (int l0 = lane + 64 * LU; l0 - lane < nch; l0 += 64 * LU) {   // uniform over the wave
    request(l0);
    merge(l0);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {             // butterfly over the wave
    float od[KL];
    int oi[KL];
#pragma unroll
    for (int e = 0; e < KL; ++e) { od[e] = __shfl_xor(bd[e], off); oi[e] = __shfl_xor(bi[e], off); }
    merge_sorted_lex(bd, bi, od, oi);
  }
  const int kt = min(k, pool);                           // k_t = min(k, |pool|) ([RKV] §2.1)
  int jj[KL];
#pragma unroll
  for (int e = 0; e < KL; ++e) jj[e] = e < kt ? bi[e] : kNoRef;
#pragma unroll
  for (int a = 1; a < KL; ++a)                           // ascending position
#pragma unroll
    for (int m = a; m > 0; --m) {
      const int lo = min(jj[m - 1], jj[m]), hi = max(jj[m - 1], jj[m]);
      jj[m - 1] = lo;
      jj[m] = hi;
    }
  if (lane == 0) {
    for (int e = 0; e < k; ++e) {
      if (writer) ref_idx[row * k + e] = e < kt ? ref_position(sv, jj[e]) : -1;
      if (e < KL) sel[e] = e < kt ? int(refs.row(b, jj[e])) : -1;   // stored row
      if (selj && e < KL) selj[e] = e < kt ? jj[e] : -1;             // reference index
    }
    if (writer && act) act[b] = 1;
  }
  return kt;
}

// Workgroup: features [16 fb, 16 fb + 16) of RB (2 or 4) appended tokens
// over the 512-row chunks s, s + S, s + 2S, ... of the C rows (S slices; the
// feature block runs fastest, then the slice).  After choosing the tokens'
// references (wave r for token r), four consecutive lanes cover the 16
// features of one row of W1 and of W2 (32 contiguous bytes each at bf16), so
// a wave's load touches 16 rows; the 64 row groups of the workgroup take 8
// consecutive rows each of a chunk.  The first chunk's W1 and W2 are
// requested during the selection and each next chunk's while the current
// one is multiplied; with two tokens, both tokens' rows of a chunk are
// requested together.  The mean of the chosen references is formed at the
// rows a thread needs, in fp32 from the stored rows (sum in order, times
// 1/k_t).  For its RB tokens a thread accumulates x.W1, x.W2, m.W1, m.W2 for
// its 4 features; the 64 partial sums of each value are reduced through LDS
// in a fixed order into the slice's partial sums
// ph[b][s][x.W1 | x.W2 | m.W1 | m.W2][d_ff].
template <typename E, int KL, bool FP8, int RB>
__global__ __launch_bounds__(256) void k_app_sel_proj(
    void* __restrict__ kv, const E* __restrict__ kv_new, const int32_t* __restrict__ pos,
    SchedView sv, int T, int C, int k, int rec_bytes, int n_groups, int d_c, int n_lists,
    const float2* __restrict__ part, int32_t* __restrict__ ref_idx, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zmin, float* __restrict__ z,
    const E* __restrict__ w1, const E* __restrict__ w2, int B, int d_ff, int S,
    float* __restrict__ ph, int* __restrict__ act) {
  constexpr int NV = RB * 16, RPT = 8, RG = 64;           // values: [token][x|m][W1|W2][feature]
  constexpr int CH = RG * RPT;                           // rows per chunk
  const int nfb = d_ff / 16;                             // feature blocks; tokens RB at a time
  const int fb = blockIdx.x % nfb, sl = (blockIdx.x / nfb) % S;
  const int b0 = (blockIdx.x / (nfb * S)) * RB;
  const int tid = threadIdx.x, fq = tid & 3, rg = tid >> 2;
  const int f0 = fb * 16 + fq * 4;                       // this lane's 4 features
  __shared__ float red[NV * (256 + 1)];
  __shared__ float tot[4 * NV];
  __shared__ int sel_l[RB][KL];
  __shared__ int kt_l[RB];
  static_assert(RB == 2 || RB == 4, "one wave selects each of the workgroup's tokens");
  // W1 and W2 of the first chunk do not depend on the selection: requested
  // during it, so their latency passes under the merge (rows past C read row
  // C - 8 and go unused)
  const int c1_first = min(sl * CH + rg * RPT, C - RPT);
  RawW4<E> wa[RPT], wb[RPT];
  auto prefetch = [&]() {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      wa[i].load(w1 + size_t(c1_first + i) * d_ff + f0);
      wb[i].load(w2 + size_t(c1_first + i) * d_ff + f0);
    }
  };
  {
    const int r = tid >> 6;                              // wave r < RB selects token r
    const int b = __builtin_amdgcn_readfirstlane(b0 + r);
    int kt = -1;
    if (r < RB && b < B)
      kt = select_token<E, KL, FP8>(kv, kv_new, pos, sv, T, C, k, rec_bytes, n_groups, d_c,
                                    n_lists, part, ref_idx, codes, scale, zmin, z, act, b,
                                    fb == 0 && sl == 0, sel_l[r], prefetch);
    else
      prefetch();
    if (r < RB && (tid & 63) == 0) kt_l[r] = kt;
  }
  __syncthreads();
  const RefRows<E, FP8> refs{kv, sv, T, C};
  {
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
    bool live[RB];
    int kt[RB];
    float inv[RB];
    int srow[RB][KL];                                    // stored rows (B*T < 2^31)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      kt[r] = kt_l[r];
      live[r] = kt[r] > 0;
      inv[r] = 1.0f / float(max(kt[r], 1));
#pragma unroll
      for (int i = 0; i < KL; ++i)                       // row 0 for a token not encoded
        srow[r][i] = live[r] ? max(sel_l[r][min(i, kt[r] - 1)], 0) : 0;
    }
    // with a token encoded here there is a reference row 0, which the
    // batched loads of a token not encoded read (and drop)
    bool any_live = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) any_live = any_live || live[r];
    for (int c0 = sl * CH; any_live && c0 < C; c0 += S * CH) {
      // rows c1 .. c1 + 7 of this thread: W1 and W2 for its 4 features
      // (requested a chunk ahead), and every token's x and its references'
      // values there, all in flight together and none under a branch (C is
      // a multiple of 8, so a thread's 8 rows are all in range or all past
      // the end)
      const int c1 = c0 + rg * RPT;
      const bool in = c1 < C;
      const int cb = in ? c1 : 0;
      float a1[RPT][4], a2[RPT][4];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        wa[i].decode(a1[i]);
        wb[i].decode(a2[i]);
      }
      if (c0 + S * CH < C) {                             // uniform: the next chunk's W
        const int cn = min(c1 + S * CH, C - RPT);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          wa[i].load(w1 + size_t(cn + i) * d_ff + f0);
          wb[i].load(w2 + size_t(cn + i) * d_ff + f0);
        }
      }
      // the chunk's contribution of token r from its decoded rows
      auto accumulate = [&](int r, const float (&xv)[RPT], const float (&v)[KL][RPT]) {
        float mv[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
          float m = 0.0f;
#pragma unroll
          for (int i = 0; i < KL; ++i)
            if (i < kt[r]) m += v[i][e];
          mv[e] = m * inv[r];
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            acc[r * 16 + 0 + f] = fmaf(xv[i], a1[i][f], acc[r * 16 + 0 + f]);
            acc[r * 16 + 4 + f] = fmaf(xv[i], a2[i][f], acc[r * 16 + 4 + f]);
            acc[r * 16 + 8 + f] = fmaf(mv[i], a1[i][f], acc[r * 16 + 8 + f]);
            acc[r * 16 + 12 + f] = fmaf(mv[i], a2[i][f], acc[r * 16 + 12 + f]);
          }
      };
      if constexpr (RB == 2) {
        // both tokens' rows requested before either is used
        RawW8<E> xr[RB];
        typename RefRows<E, FP8>::Raw rr[RB][KL];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          xr[r].load(kv_new + size_t(min(b0 + r, B - 1)) * C + cb);
#pragma unroll
          for (int i = 0; i < KL; ++i) refs.load_raw(size_t(srow[r][i]), cb, rr[r][i]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (!live[r] || !in) continue;                 // uniform per workgroup
          float xv[RPT], v[KL][RPT];
          xr[r].decode(xv);
#pragma unroll
          for (int i = 0; i < KL; ++i) rr[r][i].decode(v[i]);
          accumulate(r, xv, v);
        }
      } else {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (!live[r] || !in) continue;                 // uniform per workgroup
          float xv[RPT], v[KL][RPT];
          load8(kv_new + size_t(b0 + r) * C + cb, xv);
#pragma unroll
          for (int i = 0; i < KL; ++i) refs.load(size_t(srow[r][i]), cb, v[i]);
          accumulate(r, xv, v);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) red[v * 257 + tid] = acc[v];
    __syncthreads();
    for (int i = tid; i < 4 * NV; i += 256) {
      // output (v, q): value v of the lanes with fq == q, summed over the
      // 64 row groups in order
      const int q = i & 3, v = i >> 2;
      float s = 0.0f;
      for (int g = 0; g < RG; ++g) s += red[v * 257 + g * 4 + q];
      tot[q * NV + v] = s;
    }
    __syncthreads();
    if (tid < RB * 16) {                                 // (token r, lane group q, feature f)
      const int r = tid / 16, q = (tid / 4) & 3, f = tid & 3;
      if (live[r]) {
        const float* u = tot + q * NV + r * 16;
        float* dst = ph + (size_t(b0 + r) * S + sl) * 4 * d_ff + fb * 16 + q * 4 + f;
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[size_t(v) * d_ff] = u[4 * v + f];
      }
    }
  }
}

// ---------------------------------------------------------------- W3 + quantiser
constexpr int kAppF = 4096;         // delta_h features the W3 kernel holds in LDS at a time

// z = delta_h W3 for columns [c0, c0 + CB) of token b, CB = 32 (g <= 32) or
// 64, then the group quantiser ([RKV] §2.4) and the record, written when
// `live` (row = b T + pos_of(), read only then and only at the end).  Over
// the features in blocks of kAppF: produce(fc,
// nf, dhl) fills dhl[0, nf) with delta_h of features [fc, fc + nf) (every
// thread takes part; the first rows of W3 of the block are already in
// flight); then LPR = CB/8 lanes cover a row of the column block, 8 columns
// each, and the 256/LPR row groups sum delta_h[f] W3[f][.] over f = rg +
// (256/LPR) i, 16 rows' loads in flight at a time; the partial rows are
// reduced in LDS; the first LPR lanes then hold 8 consecutive latents each
// and run the quantiser.
constexpr int kW3Un = 16;          // W3 rows in flight per thread

// The first block's W3 rows of a thread of w3_quantise, for a caller that
// requests them early (PRE).
template <typename E, int CB>
__device__ __forceinline__ void w3_first_rows(RawW8<E> (&wr)[kW3Un], const E* __restrict__ w3,
                                              int c0, int d_ff, int d_c) {
  constexpr int LPR = CB / 8, RG = 256 / LPR;
  const int tid = threadIdx.x, cg = tid % LPR, rg = tid / LPR;
  const int nf = min(kAppF, d_ff);
#pragma unroll
  for (int u = 0; u < kW3Un; ++u) wr[u].load(w3 + c0 + cg * 8 + size_t(min(rg + RG * u, nf - 1)) * d_c);
}

template <typename E, int BITS, int G8, int CB, bool PRE, typename Produce, typename PosOf>
__device__ __forceinline__ void w3_quantise(int b, int c0, bool live, PosOf pos_of, int T, int d_ff,
                                            int d_c, const E* __restrict__ w3,
                                            uint8_t* __restrict__ codes,
                                            uint16_t* __restrict__ scale,
                                            uint16_t* __restrict__ zmin, float* __restrict__ z,
                                            Produce produce, RawW8<E> (&wr)[kW3Un]) {
  constexpr int LPR = CB / 8, RG = 256 / LPR, UN = kW3Un;
  const int tid = threadIdx.x, cg = tid % LPR, rg = tid / LPR;
  __shared__ float red[RG * (CB + 1)];
  __shared__ float zl[CB];
  __shared__ float dhl[kAppF];
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const E* wcol = w3 + c0 + cg * 8;
  for (int fc = 0; fc < d_ff; fc += kAppF) {
    const int nf = min(kAppF, d_ff - fc);                // a multiple of 16
    if (!PRE || fc > 0)                                  // (PRE: the first block's came in wr)
#pragma unroll
      for (int u = 0; u < UN; ++u) wr[u].load(wcol + size_t(fc + min(rg + RG * u, nf - 1)) * d_c);
    produce(fc, nf, dhl);
    __syncthreads();
    for (int f1 = rg; f1 < nf; f1 += RG * UN) {
      if (f1 != rg)
#pragma unroll
        for (int u = 0; u < UN; ++u) wr[u].load(wcol + size_t(fc + min(f1 + RG * u, nf - 1)) * d_c);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float d = f1 + RG * u < nf ? dhl[f1 + RG * u] : 0.0f;
        float w[8];
        wr[u].decode(w);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(d, w[e], acc[e]);
      }
    }
    __syncthreads();                                     // dhl is rewritten by the next block
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * (CB + 1) + cg * 8 + e] = acc[e];
  __syncthreads();
  if (tid < CB) {
    float s = 0.0f;
    for (int r = 0; r < RG; ++r) s += red[r * (CB + 1) + tid];
    zl[tid] = s;
  }
  __syncthreads();
  if (tid < 64) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tid < LPR ? zl[min(tid, LPR - 1) * 8 + e] : 0.0f;
    const size_t row = size_t(b) * T + (live ? pos_of() : 0);
    const int64_t unit = int64_t(row) * (d_c / 8) + c0 / 8 + tid;
    write_record8<BITS, G8>(v, live && tid < LPR, tid, unit, codes, scale, zmin);
    if (live && tid < LPR) {
      if (z) {
        float4* dst = reinterpret_cast<float4*>(z + unit * 8);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// Workgroup (token b, columns [CB*w, CB*w + CB)): delta_h of each block of
// features formed in LDS from the S slices' partial sums (added in slice
// order, [RKV] §2.3), then w3_quantise.  No early exit: the loads go out
// together with the act flag's, and a token not encoded (a reference, or no
// append) only has its writes skipped (its partial sums were not written;
// they are read in bounds and their results dropped).
template <typename E, int BITS, int G8, int CB>
__global__ __launch_bounds__(256) void k_app_w3(const float* __restrict__ ph, int S,
                                                const int* __restrict__ act,
                                                const int32_t* __restrict__ pos,
                                                const E* __restrict__ w3, int T, int d_ff,
                                                int d_c, uint8_t* __restrict__ codes,
                                                uint16_t* __restrict__ scale,
                                                uint16_t* __restrict__ zmin,
                                                float* __restrict__ z) {
  const int nblk = d_c / CB;
  const int b = blockIdx.x / nblk, c0 = (blockIdx.x % nblk) * CB;
  const bool live = act[b] == 1;
  const float* phb = ph + size_t(b) * S * 4 * d_ff;
  auto produce = [&](int fc, int nf, float* dhl) {
    for (int f = threadIdx.x * 4; f < nf; f += 256 * 4) {
      // four slices' loads in flight at once, added in slice order (a
      // slice past the last re-reads the last and is not added)
      float4 a[4];
      auto batch = [&](int s0) {
        float4 t4[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            t4[j][v] = *reinterpret_cast<const float4*>(
                phb + size_t(4 * min(s0 + j, S - 1) + v) * d_ff + fc + f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool first = s0 + j == 0, add = s0 + j > 0 && s0 + j < S;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            a[v].x = first ? t4[j][v].x : (add ? a[v].x + t4[j][v].x : a[v].x);
            a[v].y = first ? t4[j][v].y : (add ? a[v].y + t4[j][v].y : a[v].y);
            a[v].z = first ? t4[j][v].z : (add ? a[v].z + t4[j][v].z : a[v].z);
            a[v].w = first ? t4[j][v].w : (add ? a[v].w + t4[j][v].w : a[v].w);
          }
        }
      };
      batch(0);
      for (int s0 = 4; s0 < S; s0 += 4) batch(s0);
      float4 o;
      o.x = silu(a[0].x) * a[1].x - silu(a[2].x) * a[3].x;
      o.y = silu(a[0].y) * a[1].y - silu(a[2].y) * a[3].y;
      o.z = silu(a[0].z) * a[1].z - silu(a[2].z) * a[3].z;
      o.w = silu(a[0].w) * a[1].w - silu(a[2].w) * a[3].w;
      *reinterpret_cast<float4*>(dhl + f) = o;
    }
  };
  RawW8<E> wr[kW3Un];
  w3_quantise<E, BITS, G8, CB, false>(b, c0, live, [&]() { return pos[b]; }, T, d_ff, d_c, w3,
                                      codes, scale, zmin, z, produce, wr);
}

// ---------------------------------------------------------------- projections of rows
// Rows of the reference-projection path: out[(v * S + sl) * 2 d_ff + o] =
// sum over the C rows c of slice sl's 512-row chunks (sl, sl + S, ...) of
// vec_v[c] [W1 | W2][c][o] in fp32, for the RB row vectors v0 .. v0 + RB - 1
// and the 16 outputs o of block ob of [W1 | W2] (a block lies in W1 or in W2:
// d_ff is a multiple of 16).  Workgroup blk = ob + (2 d_ff / 16) (sl + S
// (v0 / RB)), the output block fastest.  Four consecutive lanes cover the
// block's 16 outputs of a row of W (32 contiguous bytes at bf16); the 64 row
// groups take 8 consecutive rows each of a chunk; the first chunk's W is
// requested first and each next chunk's while the current one is
// multiplied; four vectors' rows are requested together.  The 64 row
// groups' partial sums are added through LDS in a fixed order.  `vecs`
// gives, for local vector r: valid(r), load(r, c, raw) (8 values at row c,
// in bounds whatever r) and decode(r, raw, v).
template <typename E, int RB, typename Vecs>
__device__ __forceinline__ void proj_block(const E* __restrict__ w1, const E* __restrict__ w2,
                                           int C, int d_ff, int S, int blk, const Vecs vecs,
                                           float* __restrict__ out) {
  constexpr int NV = RB * 4, RPT = 8, RG = 64, CH = RG * RPT, TB = 4;
  static_assert(RB % TB == 0, "vectors in batches of four");
  const int nob = 2 * d_ff / 16;
  const int ob = blk % nob, sl = (blk / nob) % S, v0 = (blk / (nob * S)) * RB;
  const int tid = threadIdx.x, fq = tid & 3, rg = tid >> 2;
  const int o0 = ob * 16 + fq * 4;                       // this lane's 4 outputs
  const E* w = o0 < d_ff ? w1 + o0 : w2 + (o0 - d_ff);
  __shared__ float red[NV * (256 + 1)];
  static_assert(RB <= 32, "one bit per vector");
  uint32_t vmask = 0;                                    // bit r: vector r is valid
#pragma unroll
  for (int r = 0; r < RB; ++r) vmask |= vecs.valid(r) ? 1u << r : 0u;
  if (vmask == 0) return;                                // uniform over the workgroup
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
  const int c1_first = min(sl * CH + rg * RPT, C - RPT);
  RawW4<E> wa[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) wa[i].load(w + size_t(c1_first + i) * d_ff);
  for (int c0 = sl * CH; c0 < C; c0 += S * CH) {
    const int c1 = c0 + rg * RPT;
    const bool in = c1 < C;                              // C is a multiple of 8
    const int cb = in ? c1 : 0;
    float a[RPT][4];
#pragma unroll
    for (int i = 0; i < RPT; ++i) wa[i].decode(a[i]);
    if (c0 + S * CH < C) {                               // uniform: the next chunk's W
      const int cn = min(c1 + S * CH, C - RPT);
#pragma unroll
      for (int i = 0; i < RPT; ++i) wa[i].load(w + size_t(cn + i) * d_ff);
    }
#pragma unroll
    for (int r0 = 0; r0 < RB; r0 += TB) {
      typename Vecs::Raw raw[TB];
#pragma unroll
      for (int u = 0; u < TB; ++u) vecs.load(r0 + u, cb, raw[u]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < TB; ++u) {
        const int r = r0 + u;
        if (!((vmask >> r) & 1u) || !in) continue;       // uniform per workgroup
        float xv[RPT];
        vecs.decode(r, raw[u], xv);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[r * 4 + f] = fmaf(xv[i], a[i][f], acc[r * 4 + f]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) red[v * 257 + tid] = acc[v];
  __syncthreads();
  const int n2 = 2 * d_ff;
  for (int i = tid; i < 4 * NV; i += 256) {
    // value v (vector v / 4, output v % 4 of a lane) of the lanes with
    // fq == q, summed over the 64 row groups in order
    const int q = i & 3, v = i >> 2, r = v >> 2, f = v & 3;
    float sum = 0.0f;
    for (int g = 0; g < RG; ++g) sum += red[v * 257 + g * 4 + q];
    if ((vmask >> r) & 1u) out[(size_t(v0 + r) * S + sl) * n2 + ob * 16 + q * 4 + f] = sum;
  }
}

// The appended tokens as row vectors: token b0 + r, valid when its position
// is in [0, T); a token whose position is a reference of an FP8 store
// enters with its E4M3 values (the values the store will hold).
template <typename E, int RB, bool FP8>
struct NewTokenVecs {
  using Raw = RawW8<E>;
  const E* kv_new;
  int C, B, b0;
  int st[RB];                                            // 0 not appended, 1 encoded, 2 reference
  __device__ bool valid(int r) const { return st[r] != 0; }
  __device__ void load(int r, int c, Raw& raw) const {
    raw.load(kv_new + size_t(min(b0 + r, B - 1)) * C + c);
  }
  __device__ void decode(int r, const Raw& raw, float (&v)[8]) const {
    raw.decode(v);
    if constexpr (FP8)
      if (st[r] == 2)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fp8_round(v[e]);
  }
};

// The stored references as row vectors: vector v0 + r = reference j of
// sequence b, v = b nref + j, valid below B nref.
template <typename E, int RB, bool FP8>
struct StoredRefVecs {
  using Raw = typename RefRows<E, FP8>::Raw;
  RefRows<E, FP8> refs;
  int nref, n_vec, v0;
  __device__ bool valid(int r) const { return v0 + r < n_vec; }
  __device__ void load(int r, int c, Raw& raw) const {
    const int v = min(v0 + r, n_vec - 1);
    refs.load_raw(refs.row(v / nref, v % nref), c, raw);
  }
  __device__ void decode(int, const Raw& raw, float (&v)[8]) const { raw.decode(v); }
};

// P[b][j] = r_j [W1 | W2] for every reference the cache holds (rkv_project_refs).
template <typename E, bool FP8>
__global__ __launch_bounds__(256) void k_ref_proj(const void* __restrict__ kv, SchedView sv,
                                                  int T, int C, int B,
                                                  const E* __restrict__ w1,
                                                  const E* __restrict__ w2, int d_ff,
                                                  float* __restrict__ ref_proj) {
  constexpr int RB = 16;
  const int nob = 2 * d_ff / 16;
  StoredRefVecs<E, RB, FP8> vecs{RefRows<E, FP8>{kv, sv, T, C}, sv.nref, B * sv.nref,
                                 int(blockIdx.x / nob) * RB};
  proj_block<E, RB>(w1, w2, C, d_ff, 1, int(blockIdx.x), vecs, ref_proj);
}

// The first launch of the append with reference projections: workgroups
// below n_dist are the distance workgroups; the rest project the appended
// tokens: px[b][sl][.] = the slice's partial sums of x [W1 | W2].
template <typename E, int KL, bool FP8, int U, int RB>
__global__ __launch_bounds__(256) void k_app_dist_xproj(
    const void* __restrict__ kv, const E* __restrict__ kv_new, const int32_t* __restrict__ pos,
    SchedView sv, int T, int C, int n_lists, float2* __restrict__ part, int n_dist,
    const E* __restrict__ w1, const E* __restrict__ w2, int d_ff, int S, int B,
    float* __restrict__ px) {
  const int blk = int(blockIdx.x);
  if (blk < n_dist) {
    dist_block<E, KL, FP8, U>(kv, kv_new, pos, sv, T, C, n_lists, part, blk);
    return;
  }
  const int w = blk - n_dist, nob = 2 * d_ff / 16;
  NewTokenVecs<E, RB, FP8> vecs{kv_new, C, B, (w / (nob * S)) * RB, {}};
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int b = vecs.b0 + r;
    int st = 0;
    if (b < B) {
      const int t = pos[b];
      if (t >= 0 && t < T) {
        bool is_ref;
        (void)refs_before(sv, t, is_ref);
        st = is_ref ? 2 : 1;
      }
    }
    vecs.st[r] = st;
  }
  proj_block<E, RB>(w1, w2, C, d_ff, S, w, vecs, px);
}

// The second launch of the append with reference projections.  Workgroup
// (token b, columns [CB w, CB w + CB)): its first wave chooses the token's
// references from the distance lists (select_token; the workgroup of the
// first column block writes ref_idx, and stores a reference token in the
// cache with a zero record and its row of P, the sum of its slices'
// partial projections in slice order).  For an encoded token, delta_h =
// Swish(x W1) (x W2) - Swish(m W1) (m W2) ([RKV] §2.3), with x [W1 | W2]
// from the slices' partial sums (in slice order) and m [W1 | W2] the mean of
// the chosen references' rows of P (the first layer of f_c is linear, so
// the projection of their mean is the mean of their projections, [RKV] §2.2
// mean eq.; summed in order, times 1/k_t); then w3_quantise.
template <typename E, int KL, bool FP8, int BITS, int G8, int CB>
__global__ __launch_bounds__(256) void k_app_sel_w3(
    void* __restrict__ kv, const E* __restrict__ kv_new, const int32_t* __restrict__ pos,
    SchedView sv, int T, int C, int k, int rec_bytes, int n_groups, int d_c, int n_lists,
    const float2* __restrict__ part, int32_t* __restrict__ ref_idx, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zmin, float* __restrict__ z,
    const float* __restrict__ px, int S, float* __restrict__ ref_proj,
    const E* __restrict__ w3, int d_ff) {
  const int nblk = d_c / CB;
  const int b = int(blockIdx.x) / nblk, c0 = (int(blockIdx.x) % nblk) * CB;
  const bool writer = c0 == 0;
  const int tid = threadIdx.x, n2 = 2 * d_ff;
  __shared__ int sel_l[KL], selj_l[KL];
  __shared__ int kt_l;
  // the first block's W3 rows do not depend on the selection: requested
  // during it (by the selecting wave right after its lists)
  RawW8<E> wr[kW3Un];
  auto pre = [&]() { w3_first_rows<E, CB>(wr, w3, c0, d_ff, d_c); };
  if (tid < 64) {
    const int bb = __builtin_amdgcn_readfirstlane(b);
    const int kt = select_token<E, KL, FP8>(kv, kv_new, pos, sv, T, C, k, rec_bytes, n_groups,
                                            d_c, n_lists, part, ref_idx, codes, scale, zmin, z,
                                            nullptr, bb, writer, sel_l, pre, selj_l);
    if (tid == 0) kt_l = kt;
  } else {
    pre();
  }
  __syncthreads();
  const int kt = kt_l;
  const float* pxb = px + size_t(b) * S * n2;
  if (kt <= 0) {                                         // not encoded
    if (writer) {
      const int t = pos[b];
      if (t >= 0 && t < T) {
        bool is_ref;
        const int j = refs_before(sv, t, is_ref);
        if (is_ref)                                      // its row of P
          for (int o = tid; o < n2; o += 256) {
            float sum = pxb[o];
            for (int s = 1; s < S; ++s) sum += pxb[size_t(s) * n2 + o];
            ref_proj[(size_t(b) * sv.nref + j) * n2 + o] = sum;
          }
      }
    }
    return;
  }
  const float inv = 1.0f / float(kt);
  int jr[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) jr[i] = max(selj_l[min(i, kt - 1)], 0);
  const float* pb = ref_proj + size_t(b) * sv.nref * n2;
  auto ld4 = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
  auto add4 = [](float4& a, const float4& t) { a.x += t.x; a.y += t.y; a.z += t.z; a.w += t.w; };
  auto produce = [&](int fc, int nf, float* dhl) {
    for (int f = tid * 4; f < nf; f += 256 * 4) {
      // every load of the 4 features in flight together: the chosen
      // references' rows of P, then the slices' partial sums
      float4 pa[KL], pm[KL];
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        pa[i] = ld4(pb + size_t(jr[i]) * n2 + fc + f);
        pm[i] = ld4(pb + size_t(jr[i]) * n2 + d_ff + fc + f);
      }
      float4 xa = ld4(pxb + fc + f), xb = ld4(pxb + d_ff + fc + f);
      for (int s = 1; s < S; ++s) {
        add4(xa, ld4(pxb + size_t(s) * n2 + fc + f));
        add4(xb, ld4(pxb + size_t(s) * n2 + d_ff + fc + f));
      }
      float4 ma = pa[0], mb = pm[0];
#pragma unroll
      for (int i = 1; i < KL; ++i)
        if (i < kt) {
          add4(ma, pa[i]);
          add4(mb, pm[i]);
        }
      float4 o;
      o.x = silu(xa.x) * xb.x - silu(ma.x * inv) * (mb.x * inv);
      o.y = silu(xa.y) * xb.y - silu(ma.y * inv) * (mb.y * inv);
      o.z = silu(xa.z) * xb.z - silu(ma.z * inv) * (mb.z * inv);
      o.w = silu(xa.w) * xb.w - silu(ma.w * inv) * (mb.w * inv);
      *reinterpret_cast<float4*>(dhl + f) = o;
    }
  };
  w3_quantise<E, BITS, G8, CB, true>(b, c0, true, [&]() { return pos[b]; }, T, d_ff, d_c, w3,
                                     codes, scale, zmin, z, produce, wr);
}

}  // namespace

// Fixed device scratch of the allocation-free append (rkv_append_noalloc):
// the same regions plan_append lays out, in a module array instead of a
// caller's workspace.  Each GPU that loads the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns for the
// current device may reach a kernel.
static __device__ __align__(256) char scratch[kAppendScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t append_scratch(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {               // once per device, with it current
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<char*>(addr);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// Slices of the C rows in the projection launch: enough that it has about
// two workgroups per compute unit (512) where the tokens and feature blocks
// alone give fewer, at most one 512-row chunk each.  More slices mean more
// partial sums to add in the W3 launch, and other sums in fp32 (the slices
// are added in order, so a shape always gives the same bits).
// RKV_APP_SPLIT=n in the environment (read at every call, the workspace
// query included) forces n slices, clamped to [1, chunks].
// Appended tokens per projection workgroup: 2 for one or two sequences
// (fewer accumulators, both tokens' rows requested together), else 4 (the
// workgroups of four tokens read each chunk of W once for all four).  In one
// process at C = 2048, d_ff = 1024: B = 1 23.3 against 24.3 us per call with
// 4; B = 16 54.3 against 53.1 us.  RKV_APP_RB=2|4 in the environment (read
// at every call, the workspace query included) forces one.
static int append_tokens_per_block(const Shape& sh) {
  if (const char* force = std::getenv("RKV_APP_RB")) return std::atoi(force) == 4 ? 4 : 2;
  return sh.B <= 2 ? 2 : 4;
}

static int append_split(const Shape& sh, int rb) {
  const int chunks = cdiv(sh.C, 512);
  const int groups = sh.d_ff / 16 * cdiv(sh.B, rb);
  int s = std::max(1, cdiv(512, groups));
  if (const char* force = std::getenv("RKV_APP_SPLIT")) s = std::atoi(force);
  return std::min(std::max(s, 1), chunks);
}

AppendWorkspace plan_append(const Shape& sh) {
  AppendWorkspace L{};
  L.n_lists = cdiv(std::max(sh.nref, 1), kAppCH);
  L.rb = append_tokens_per_block(sh);
  L.n_split = append_split(sh, L.rb);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.rpos = take(size_t(sh.nref) * 4);
  L.part = take(size_t(sh.B) * L.n_lists * sh.kl * 8);
  L.ph = take(size_t(sh.B) * L.n_split * 4 * sh.d_ff * 4);
  L.act = take(size_t(sh.B) * 4);
  L.total = off;
  return L;
}

hipError_t launch_append(const Shape& sh, void* kv, const void* kv_new, const int32_t* pos,
                         const void* w1, const void* w2, const void* w3, int32_t* ref_idx,
                         uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z, char* ws,
                         const AppendWorkspace& L, hipStream_t st) {
  SchedView sv{nullptr, sh.nref, sh.s, sh.n_sink};
  if (sh.alpha != 0.0) {
    int* rpos = reinterpret_cast<int*>(ws + L.rpos);
    const hipError_t e = launch_ref_positions(sh, rpos, st);
    if (e != hipSuccess) return e;
    sv.rpos = rpos;
  }
  auto* part = reinterpret_cast<float2*>(ws + L.part);
  auto* ph = reinterpret_cast<float*>(ws + L.ph);
  auto* act = reinterpret_cast<int*>(ws + L.act);
  const int rec_bytes = sh.d_c * sh.b / 8;
  const int n_groups = sh.b == kIdentityBits ? 0 : sh.d_c / sh.g;   // identity: no group numbers
  const int cb = sh.g <= 32 || sh.b == kIdentityBits ? 32 : 64;   // a block holds whole groups
  const int n_dist = sh.B * L.n_lists;
  // coordinates per lane in flight in the distance launch: 4 x 8 where it
  // has at most two workgroups per compute unit (its time is then the
  // latency of one batch), 2 x 8 above (more waves fit, which a launch
  // bound by HBM bandwidth prefers).  RKV_APP_DIST_U=2|4 in the environment
  // forces one; both give the same bits.
  int dist_u = n_dist <= 512 ? 4 : 2;
  if (const char* force = std::getenv("RKV_APP_DIST_U")) dist_u = std::atoi(force) == 4 ? 4 : 2;

#define RKV_APP(E, KL, F8)                                                                        \
  if (dist_u == 4)                                                                                \
    k_app_dist<E, KL, F8, 4><<<n_dist, 256, 0, st>>>(kv, static_cast<const E*>(kv_new), pos, sv,  \
                                                     sh.T, sh.C, L.n_lists, part);               \
  else                                                                                            \
    k_app_dist<E, KL, F8, 2><<<n_dist, 256, 0, st>>>(kv, static_cast<const E*>(kv_new), pos, sv,  \
                                                     sh.T, sh.C, L.n_lists, part);               \
  if (L.rb == 2)                                                                                   \
    k_app_sel_proj<E, KL, F8, 2><<<sh.d_ff / 16 * L.n_split * cdiv(sh.B, 2), 256, 0, st>>>(        \
        kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, sh.k, rec_bytes, n_groups, sh.d_c, \
        L.n_lists, part, ref_idx, codes, scale, zmin, z, static_cast<const E*>(w1),            \
        static_cast<const E*>(w2), sh.B, sh.d_ff, L.n_split, ph, act);                         \
  else                                                                                            \
    k_app_sel_proj<E, KL, F8, 4><<<sh.d_ff / 16 * L.n_split * cdiv(sh.B, 4), 256, 0, st>>>(        \
        kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, sh.k, rec_bytes, n_groups, sh.d_c, \
        L.n_lists, part, ref_idx, codes, scale, zmin, z, static_cast<const E*>(w1),            \
        static_cast<const E*>(w2), sh.B, sh.d_ff, L.n_split, ph, act)
#define RKV_APPK(E, F8) \
  if (sh.kl == 4) { RKV_APP(E, 4, F8); } else { RKV_APP(E, 8, F8); }
  if (sh.bf16) {
    if (sh.ref_fp8) { RKV_APPK(uint16_t, true) } else { RKV_APPK(uint16_t, false) }
  } else {
    if (sh.ref_fp8) { RKV_APPK(float, true) } else { RKV_APPK(float, false) }
  }
#undef RKV_APPK
#undef RKV_APP

  const int n_w3 = sh.B * (sh.d_c / cb);
#define RKV_W3(E, BITS, G8)                                                                        \
  if (cb == 32)                                                                                    \
    k_app_w3<E, BITS, G8, 32><<<n_w3, 256, 0, st>>>(ph, L.n_split, act, pos, static_cast<const E*>(w3),      \
                                                    sh.T, sh.d_ff, sh.d_c, codes, scale, zmin, z); \
  else                                                                                             \
    k_app_w3<E, BITS, G8, 64><<<n_w3, 256, 0, st>>>(ph, L.n_split, act, pos, static_cast<const E*>(w3),      \
                                                    sh.T, sh.d_ff, sh.d_c, codes, scale, zmin, z)
#define RKV_W3G(E, BITS)                   \
  switch (sh.g) {                          \
    case 8: RKV_W3(E, BITS, 1); break;     \
    case 16: RKV_W3(E, BITS, 2); break;    \
    case 32: RKV_W3(E, BITS, 4); break;    \
    default: RKV_W3(E, BITS, 8); break;    \
  }
  if (sh.bf16) {
    if (sh.b == 4) { RKV_W3G(uint16_t, 4) } else if (sh.b == 2) { RKV_W3G(uint16_t, 2) }
    else { RKV_W3(uint16_t, kIdentityBits, 1); }
  } else {
    if (sh.b == 4) { RKV_W3G(float, 4) } else if (sh.b == 2) { RKV_W3G(float, 2) }
    else { RKV_W3(float, kIdentityBits, 1); }
  }
#undef RKV_W3G
#undef RKV_W3
  return hipGetLastError();
}

// ---------------------------------------------------------------- with reference projections
// Slices of the C rows in the token projection of the first launch: about
// 512 projection workgroups where the output blocks and token blocks alone
// give fewer, at most one 512-row chunk each (RKV_APP_SPLIT=n forces n, as
// for rkv_append).
static int append_proj_split(const Shape& sh) {
  const int chunks = cdiv(sh.C, 512);
  int s = std::max(1, cdiv(512, 2 * sh.d_ff / 16 * cdiv(sh.B, 4)));
  if (const char* force = std::getenv("RKV_APP_SPLIT")) s = std::atoi(force);
  return std::min(std::max(s, 1), chunks);
}

AppendWorkspace plan_append_proj(const Shape& sh) {
  AppendWorkspace L{};
  L.n_lists = cdiv(std::max(sh.nref, 1), kAppCH);
  L.n_split = append_proj_split(sh);
  L.rb = 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.rpos = take(size_t(sh.nref) * 4);
  L.part = take(size_t(sh.B) * L.n_lists * sh.kl * 8);
  L.ph = take(size_t(sh.B) * L.n_split * 2 * sh.d_ff * 4);   // x [W1 | W2] partial sums
  L.act = take(0);
  L.total = std::max<size_t>(off, 256);
  return L;
}

static hipError_t sched_view(const Shape& sh, char* ws, const AppendWorkspace& L, hipStream_t st,
                             SchedView& sv) {
  sv = SchedView{nullptr, sh.nref, sh.s, sh.n_sink};
  if (sh.alpha != 0.0) {
    int* rpos = reinterpret_cast<int*>(ws + L.rpos);
    const hipError_t e = launch_ref_positions(sh, rpos, st);
    if (e != hipSuccess) return e;
    sv.rpos = rpos;
  }
  return hipSuccess;
}

AppendWorkspace plan_project_refs(const Shape& sh) {
  AppendWorkspace L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.rpos = take(size_t(sh.nref) * 4);
  L.ph = take(ref_proj_pack_bytes(sh));                  // packed W1 | W2 (matrix-core form)
  L.total = std::max<size_t>(off, 256);
  return L;
}

hipError_t launch_project_refs(const Shape& sh, const void* kv, const void* w1, const void* w2,
                               float* ref_proj, char* ws, const AppendWorkspace& L,
                               hipStream_t st) {
  if (sh.nref == 0) return hipGetLastError();
  SchedView sv;
  const hipError_t e = sched_view(sh, ws, L, st, sv);
  if (e != hipSuccess) return e;
  if (ref_proj_pack_bytes(sh) > 0 && std::getenv("RKV_REF_PROJ_VALU") == nullptr)
    return launch_ref_proj_mfma(sh, kv, w1, w2, sv, ws + L.ph, ref_proj, st);
  const int grid = 2 * sh.d_ff / 16 * cdiv(long(sh.B) * sh.nref, 16);
#define RKV_RP(E, F8)                                                                             \
  k_ref_proj<E, F8><<<grid, 256, 0, st>>>(kv, sv, sh.T, sh.C, sh.B, static_cast<const E*>(w1),    \
                                          static_cast<const E*>(w2), sh.d_ff, ref_proj)
  if (sh.bf16) {
    if (sh.ref_fp8) RKV_RP(uint16_t, true); else RKV_RP(uint16_t, false);
  } else {
    if (sh.ref_fp8) RKV_RP(float, true); else RKV_RP(float, false);
  }
#undef RKV_RP
  return hipGetLastError();
}

hipError_t launch_append_proj(const Shape& sh, void* kv, float* ref_proj, const void* kv_new,
                              const int32_t* pos, const void* w1, const void* w2, const void* w3,
                              int32_t* ref_idx, uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                              float* z, char* ws, const AppendWorkspace& L, hipStream_t st) {
  SchedView sv;
  hipError_t e = sched_view(sh, ws, L, st, sv);
  if (e != hipSuccess) return e;
  auto* part = reinterpret_cast<float2*>(ws + L.part);
  auto* px = reinterpret_cast<float*>(ws + L.ph);
  const int rec_bytes = sh.d_c * sh.b / 8;
  const int n_groups = sh.b == kIdentityBits ? 0 : sh.d_c / sh.g;
  const int n_dist = sh.B * L.n_lists;
  const int n_xp = 2 * sh.d_ff / 16 * L.n_split * cdiv(sh.B, 4);
  int dist_u = n_dist <= 512 ? 4 : 2;                    // as in rkv_append
  if (const char* force = std::getenv("RKV_APP_DIST_U")) dist_u = std::atoi(force) == 4 ? 4 : 2;
#define RKV_A1(E, KL, F8)                                                                        \
  if (dist_u == 4)                                                                               \
    k_app_dist_xproj<E, KL, F8, 4, 4><<<n_dist + n_xp, 256, 0, st>>>(                            \
        kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, L.n_lists, part, n_dist,        \
        static_cast<const E*>(w1), static_cast<const E*>(w2), sh.d_ff, L.n_split, sh.B, px);    \
  else                                                                                           \
    k_app_dist_xproj<E, KL, F8, 2, 4><<<n_dist + n_xp, 256, 0, st>>>(                            \
        kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, L.n_lists, part, n_dist,        \
        static_cast<const E*>(w1), static_cast<const E*>(w2), sh.d_ff, L.n_split, sh.B, px)
#define RKV_A1K(E, F8) \
  if (sh.kl == 4) { RKV_A1(E, 4, F8); } else { RKV_A1(E, 8, F8); }
  if (sh.bf16) {
    if (sh.ref_fp8) { RKV_A1K(uint16_t, true) } else { RKV_A1K(uint16_t, false) }
  } else {
    if (sh.ref_fp8) { RKV_A1K(float, true) } else { RKV_A1K(float, false) }
  }
#undef RKV_A1K
#undef RKV_A1
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // a workgroup's columns hold whole groups: 64 for g = 64, else 32
  const int cb = sh.g <= 32 || sh.b == kIdentityBits ? 32 : 64;
  const int n_w3 = sh.B * (sh.d_c / cb);
#define RKV_A2(E, KL, F8, BITS, G8)                                                              \
  k_app_sel_w3<E, KL, F8, BITS, G8, (G8 == 8 ? 64 : 32)><<<n_w3, 256, 0, st>>>(                  \
      kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, sh.k, rec_bytes, n_groups, sh.d_c, \
      L.n_lists, part, ref_idx, codes, scale, zmin, z, px, L.n_split, ref_proj,                  \
      static_cast<const E*>(w3), sh.d_ff)
#define RKV_A2G(E, KL, F8, BITS)            \
  switch (sh.g) {                           \
    case 8: RKV_A2(E, KL, F8, BITS, 1); break;  \
    case 16: RKV_A2(E, KL, F8, BITS, 2); break; \
    case 32: RKV_A2(E, KL, F8, BITS, 4); break; \
    default: RKV_A2(E, KL, F8, BITS, 8); break; \
  }
#define RKV_A2B(E, KL, F8)                                                              \
  if (sh.b == 4) { RKV_A2G(E, KL, F8, 4) } else if (sh.b == 2) { RKV_A2G(E, KL, F8, 2) } \
  else { RKV_A2(E, KL, F8, kIdentityBits, 1); }
#define RKV_A2K(E, F8) \
  if (sh.kl == 4) { RKV_A2B(E, 4, F8) } else { RKV_A2B(E, 8, F8) }
  if (sh.bf16) {
    if (sh.ref_fp8) { RKV_A2K(uint16_t, true) } else { RKV_A2K(uint16_t, false) }
  } else {
    if (sh.ref_fp8) { RKV_A2K(float, true) } else { RKV_A2K(float, false) }
  }
#undef RKV_A2K
#undef RKV_A2B
#undef RKV_A2G
#undef RKV_A2
  return hipGetLastError();
}

}  // namespace rkv
