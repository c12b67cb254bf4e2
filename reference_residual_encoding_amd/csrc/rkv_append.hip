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
//   sel_proj one workgroup per 16 features (and 4 tokens): each merges its
//            tokens' lists by (distance, position) itself, then x W1, x W2,
//            m W1, m W2 over all C rows (the mean m of the chosen references
//            formed in fp32 at the rows it needs), reduced in LDS, then
//            delta_h = Swish(x W1) (x W2) - Swish(m W1) (m W2) ([RKV] §2.3);
//            the first feature block writes ref_idx, and stores a reference
//            token in the cache with a zero record
//   w3       one workgroup per (token, 32 or 64 latent columns): z =
//            delta_h W3 (W3 is linear, so f_c(kv) - f_c(m) = (h(kv) - h(m))
//            W3), then the group quantiser of [RKV] §2.4 and the record
#include "rkv_device.h"
#include "rkv_internal.h"
#include "rkv_quant.h"

#include <cfloat>
#include <mutex>

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

template <typename E>
__device__ __forceinline__ void load4(const E* p, float (&v)[4]) {
  if constexpr (sizeof(E) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

template <typename E>
__device__ __forceinline__ float load1(const E* p) {
  if constexpr (sizeof(E) == 2) return bf16_to_f32(*p);
  else return *p;
}

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
  // 8 coordinates [o, o + 8) of stored row `r` (from row())
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

// State of sequence b's new token: -1 nothing to encode (invalid position
// or a reference), else the size of its pool.
__device__ __forceinline__ int pool_of(const SchedView& v, const int32_t* pos, int b, int T,
                                       int& t) {
  t = pos[b];
  if (t < 0 || t >= T) return -1;
  bool is_ref;
  const int n = refs_before(v, t, is_ref);
  return is_ref ? -1 : n;
}

// ---------------------------------------------------------------- distance
// Workgroup (b, c): pool references j in [8c, 8c + 8) of sequence b, two
// per wave with both rows' loads in flight; d = sum (x - y)^2 in fp32.
template <typename E, int KL, bool FP8>
__global__ __launch_bounds__(256) void k_app_dist(const void* __restrict__ kv,
                                                  const E* __restrict__ kv_new,
                                                  const int32_t* __restrict__ pos, SchedView sv,
                                                  int T, int C, int n_lists,
                                                  float2* __restrict__ part) {
  const RefRows<E, FP8> refs{kv, sv, T, C};
  const int b = blockIdx.x / n_lists, c = blockIdx.x % n_lists;
  int t;
  const int pool = pool_of(sv, pos, b, T, t);
  const int j0 = c * kAppCH;
  if (pool < 0 || j0 >= pool) return;
  __shared__ float dl[kAppCH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ja = j0 + 2 * wave, jb = ja + 1;
  const bool va = ja < pool, vb = jb < pool;
  const E* x = kv_new + size_t(b) * C;
  const size_t ya = refs.row(b, va ? ja : j0), yb = refs.row(b, vb ? jb : j0);
  float sa = 0.0f, sb = 0.0f;
#pragma unroll 4
  for (int o = lane * 8; o < C; o += 512) {
    float xv[8], av[8], bv[8];
    load8(x + o, xv);
    refs.load(ya, o, av);
    refs.load(yb, o, bv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float da = xv[e] - av[e], db = xv[e] - bv[e];
      sa = fmaf(da, da, sa);
      sb = fmaf(db, db, sb);
    }
  }
  sa = wave_sum(sa);
  sb = wave_sum(sb);
  if (lane == 0) {
    dl[2 * wave] = va ? sa : FLT_MAX;
    dl[2 * wave + 1] = vb ? sb : FLT_MAX;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bd[KL];
    int bi[KL];
#pragma unroll
    for (int e = 0; e < KL; ++e) { bd[e] = FLT_MAX; bi[e] = kNoRef; }
    for (int i = 0; i < kAppCH && j0 + i < pool; ++i) topk_push_lex(bd, bi, dl[i], j0 + i);
    float2* dst = part + size_t(blockIdx.x) * KL;
#pragma unroll
    for (int e = 0; e < KL; ++e) dst[e] = make_float2(bd[e], __int_as_float(bi[e]));
  }
}

// ---------------------------------------------------------------- select + projection
// One launch does both: every workgroup (16 features of RB appended tokens)
// first chooses its tokens' references itself, from the distance lists
// (they are small and L2-resident), so no launch waits for a separate
// selection.  Workgroups with fb == 0 also write the token's ref_idx, store
// a reference token as it is (with a zero record) and set act[b] = 1 when
// the token is to be encoded.
//
// Selection of sequence b's token by one wave: every lane merges the lists
// l, l + 64, ... of the ceil(pool/8) lists, then the lanes' lists are merged
// by a butterfly over the wave; by (distance, position), which orders every
// candidate uniquely, so the kept k_t = min(k, |pool|) ([RKV] §2.1) do not
// depend on the merge order.  Writes the chosen stored rows (ascending
// position) to sel[0..KL) and returns k_t; -1 when the token is not encoded
// (no append this call, or a reference).  With `writer`, also writes
// ref_idx and act[b], and stores a reference token as it is.
template <typename E, int KL, bool FP8>
__device__ int select_token(void* kv, const E* kv_new, const int32_t* pos, SchedView sv, int T,
                            int C, int k, int rec_bytes, int n_groups, int d_c, int n_lists,
                            const float2* part, int32_t* ref_idx, uint8_t* codes, uint16_t* scale,
                            uint16_t* zmin, float* z, int* act, int b, bool writer, int* sel) {
  const int lane = threadIdx.x & 63;
  const int t = pos[b];
  if (t < 0 || t >= T) {                                 // not appended this call
    if (writer && lane == 0) act[b] = 0;
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
    if (lane == 0) act[b] = 0;
    return -1;
  }
  const int nch = (pool + kAppCH - 1) / kAppCH;
  float bd[KL];
  int bi[KL];
#pragma unroll
  for (int e = 0; e < KL; ++e) { bd[e] = FLT_MAX; bi[e] = kNoRef; }
  for (int l = lane; l < nch; l += 64) {
    const float4* src = reinterpret_cast<const float4*>(part + (size_t(b) * n_lists + l) * KL);
    float4 w[KL / 2];
#pragma unroll
    for (int e = 0; e < KL / 2; ++e) w[e] = src[e];      // the whole list in flight at once
#pragma unroll
    for (int e = 0; e < KL / 2; ++e) {
      topk_push_lex(bd, bi, w[e].x, __float_as_int(w[e].y));
      topk_push_lex(bd, bi, w[e].z, __float_as_int(w[e].w));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {             // butterfly over the wave
    float od[KL];
    int oi[KL];
#pragma unroll
    for (int e = 0; e < KL; ++e) { od[e] = __shfl_xor(bd[e], off); oi[e] = __shfl_xor(bi[e], off); }
#pragma unroll
    for (int e = 0; e < KL; ++e) topk_push_lex(bd, bi, od[e], oi[e]);
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
    }
    if (writer) act[b] = 1;
  }
  return kt;
}

// Workgroup: features [16w, 16w + 16) of RB appended tokens (the feature
// block runs fastest, so the workgroups of one block of W share it in L2).
// After choosing the tokens' references, four consecutive lanes cover the
// 16 features of one row of W1 and of W2 (32 contiguous bytes each at
// bf16), so a wave's load touches 16 rows; the 64 row groups of the
// workgroup take 8 consecutive rows each of every 512-row chunk, the loads
// of a chunk in flight together.  The mean of the chosen references is
// formed at the rows a thread needs, in fp32 from the stored rows (sum in
// order, times 1/k_t).  For its RB tokens a thread accumulates x.W1, x.W2,
// m.W1, m.W2 for its 4 features; the 64 partial sums of each value are
// reduced through LDS in a fixed order, then
// delta_h = Swish(x W1) (x W2) - Swish(m W1) (m W2) ([RKV] §2.3).
template <typename E, int KL, bool FP8>
__global__ __launch_bounds__(256) void k_app_sel_proj(
    void* __restrict__ kv, const E* __restrict__ kv_new, const int32_t* __restrict__ pos,
    SchedView sv, int T, int C, int k, int rec_bytes, int n_groups, int d_c, int n_lists,
    const float2* __restrict__ part, int32_t* __restrict__ ref_idx, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zmin, float* __restrict__ z,
    const E* __restrict__ w1, const E* __restrict__ w2, int B, int d_ff,
    float* __restrict__ dh, int* __restrict__ act) {
  constexpr int RB = 4, NV = RB * 16, RPT = 8, RG = 64;  // values: [token][x|m][W1|W2][feature]
  const int nfb = d_ff / 16;                             // feature blocks; tokens RB at a time
  const int fb = blockIdx.x % nfb, b0 = (blockIdx.x / nfb) * RB;
  const int tid = threadIdx.x, fq = tid & 3, rg = tid >> 2;
  const int f0 = fb * 16 + fq * 4;                       // this lane's 4 features
  __shared__ float red[NV * (256 + 1)];
  __shared__ float tot[4 * NV];
  __shared__ int sel_l[RB][KL];
  __shared__ int kt_l[RB];
  static_assert(RB == 4, "one wave selects each of the workgroup's tokens");
  {
    const int r = tid >> 6, b = b0 + r;                  // wave r selects token r
    int kt = -1;
    if (b < B)
      kt = select_token<E, KL, FP8>(kv, kv_new, pos, sv, T, C, k, rec_bytes, n_groups, d_c,
                                    n_lists, part, ref_idx, codes, scale, zmin, z, act, b,
                                    fb == 0, sel_l[r]);
    if ((tid & 63) == 0) kt_l[r] = kt;
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
    size_t srow[RB][KL];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      kt[r] = kt_l[r];
      live[r] = kt[r] > 0;
      inv[r] = 1.0f / float(max(kt[r], 1));
#pragma unroll
      for (int i = 0; i < KL; ++i) srow[r][i] = size_t(max(sel_l[r][min(i, max(kt[r], 1) - 1)], 0));
    }
    for (int c0 = 0; c0 < C; c0 += RG * RPT) {
      // rows c1 .. c1 + 7 of this thread: W1 and W2 for its 4 features, and
      // every token's x and its references' values there, all in flight
      // together and none under a branch (C is a multiple of 8, so a
      // thread's 8 rows are all in range or all past the end)
      const int c1 = c0 + rg * RPT;
      const bool in = c1 < C;
      const int cb = in ? c1 : 0;
      float a1[RPT][4], a2[RPT][4];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        load4(w1 + size_t(cb + i) * d_ff + f0, a1[i]);
        load4(w2 + size_t(cb + i) * d_ff + f0, a2[i]);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (!live[r] || !in) continue;                   // uniform per workgroup
        float xv[RPT], mv[RPT], v[KL][RPT];
        load8(kv_new + size_t(b0 + r) * C + cb, xv);
#pragma unroll
        for (int i = 0; i < KL; ++i) refs.load(srow[r][i], cb, v[i]);
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
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) red[v * 257 + tid] = acc[v];
    __syncthreads();
    {
      // output (v, q): value v of the lanes with fq == q, summed over the
      // 64 row groups in order
      const int q = tid & 3, v = tid >> 2;
      float s = 0.0f;
      for (int g = 0; g < RG; ++g) s += red[v * 257 + g * 4 + q];
      tot[q * NV + v] = s;
    }
    __syncthreads();
    if (tid < RB * 16) {                                 // (token r, lane group q, feature f)
      const int r = tid / 16, q = (tid / 4) & 3, f = tid & 3;
      if (live[r]) {
        const float* u = tot + q * NV + r * 16;
        const float hk = silu(u[0 + f]) * u[4 + f];
        const float hm = silu(u[8 + f]) * u[12 + f];
        dh[size_t(b0 + r) * d_ff + fb * 16 + q * 4 + f] = hk - hm;
      }
    }
  }
}

// ---------------------------------------------------------------- W3 + quantiser
// Workgroup (token b, columns [CB*w, CB*w + CB)), CB = 32 (g <= 32) or 64:
// LPR = CB/8 lanes cover a row of the block, 8 columns each; the 256/LPR
// row groups sum delta_h[f] W3[f][.] over f = rg + (256/LPR) i, 16 rows'
// loads in flight at a time; the partial rows are reduced in LDS; the first
// LPR lanes then hold 8 consecutive latents each and run the group
// quantiser ([RKV] §2.4).
template <typename E, int BITS, int G8, int CB>
__global__ __launch_bounds__(256) void k_app_w3(const float* __restrict__ dh,
                                                const int* __restrict__ act,
                                                const int32_t* __restrict__ pos,
                                                const E* __restrict__ w3, int T, int d_ff,
                                                int d_c, uint8_t* __restrict__ codes,
                                                uint16_t* __restrict__ scale,
                                                uint16_t* __restrict__ zmin,
                                                float* __restrict__ z) {
  constexpr int LPR = CB / 8, RG = 256 / LPR, UN = 16;
  const int nblk = d_c / CB;
  const int b = blockIdx.x / nblk, c0 = (blockIdx.x % nblk) * CB;
  if (act[b] != 1) return;
  const int tid = threadIdx.x, cg = tid % LPR, rg = tid / LPR;
  __shared__ float red[RG * (CB + 1)];
  __shared__ float zl[CB];
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const float* dhb = dh + size_t(b) * d_ff;
  const E* wcol = w3 + c0 + cg * 8;
  for (int f1 = rg; f1 < d_ff; f1 += RG * UN) {
    float d[UN], w[UN][8];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int f = min(f1 + RG * u, d_ff - 1);
      d[u] = f1 + RG * u < d_ff ? dhb[f] : 0.0f;
      load8(wcol + size_t(f) * d_c, w[u]);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(d[u], w[u][e], acc[e]);
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
    const size_t row = size_t(b) * T + pos[b];
    const int64_t unit = int64_t(row) * (d_c / 8) + c0 / 8 + tid;
    write_record8<BITS, G8>(v, tid < LPR, tid, unit, codes, scale, zmin);
    if (tid < LPR) {
      if (z) {
        float4* dst = reinterpret_cast<float4*>(z + unit * 8);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
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

AppendWorkspace plan_append(const Shape& sh) {
  AppendWorkspace L{};
  L.n_lists = cdiv(std::max(sh.nref, 1), kAppCH);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align256(bytes); return at; };
  L.rpos = take(size_t(sh.nref) * 4);
  L.part = take(size_t(sh.B) * L.n_lists * sh.kl * 8);
  L.dh = take(size_t(sh.B) * sh.d_ff * 4);
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
  auto* dh = reinterpret_cast<float*>(ws + L.dh);
  auto* act = reinterpret_cast<int*>(ws + L.act);
  const int rec_bytes = sh.d_c * sh.b / 8;
  const int n_groups = sh.b == kIdentityBits ? 0 : sh.d_c / sh.g;   // identity: no group numbers
  const int cb = sh.g <= 32 || sh.b == kIdentityBits ? 32 : 64;   // a block holds whole groups
  const int n_dist = sh.B * L.n_lists;

#define RKV_APP(E, KL, F8)                                                                        \
  k_app_dist<E, KL, F8><<<n_dist, 256, 0, st>>>(kv, static_cast<const E*>(kv_new), pos, sv, sh.T, \
                                                sh.C, L.n_lists, part);                          \
  k_app_sel_proj<E, KL, F8><<<sh.d_ff / 16 * cdiv(sh.B, 4), 256, 0, st>>>(                         \
      kv, static_cast<const E*>(kv_new), pos, sv, sh.T, sh.C, sh.k, rec_bytes, n_groups, sh.d_c, \
      L.n_lists, part, ref_idx, codes, scale, zmin, z, static_cast<const E*>(w1),              \
      static_cast<const E*>(w2), sh.B, sh.d_ff, dh, act)
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
    k_app_w3<E, BITS, G8, 32><<<n_w3, 256, 0, st>>>(dh, act, pos, static_cast<const E*>(w3),      \
                                                    sh.T, sh.d_ff, sh.d_c, codes, scale, zmin, z); \
  else                                                                                             \
    k_app_w3<E, BITS, G8, 64><<<n_w3, 256, 0, st>>>(dh, act, pos, static_cast<const E*>(w3),      \
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

}  // namespace rkv
