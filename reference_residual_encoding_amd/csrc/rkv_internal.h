// Host-side interface between the ABI layer (rkv_api.cpp) and the kernel
// launchers (rkv_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace rkv {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int cdiv(long a, long b) { return int((a + b - 1) / b); }

// Reference schedule of one sequence ([RKV] §2.6), computed on the host.
struct Schedule {
  int T = -1, s0 = 0, n_sink = 0;
  double alpha = 0.0;
  std::vector<int> rpos;   // reference positions, ascending
  std::vector<int> nrp;    // position of the q-th non-reference token
};
// The schedule for these parameters (cached per thread).
const Schedule& schedule_for(int T, int s0, double alpha, int n_sink);

// Derived sizes of one encode problem.
struct Shape {
  int B, T, C, d_ff, d_c, k, g, b, s;
  bool bf16;
  int esize;     // bytes per kv / weight element
  int nref;      // references per sequence under the schedule
  int nr;        // non-references per sequence, T - nref
  int kl;        // neighbour-list length kept per chunk (4 or 8, >= k)
  int dist_tiling;  // the distance launch's tiling: 0 wide, 1 narrow, 2 narrow on 128-reference chunks
  int dist_bm;     // references per chunk of that tiling
  int n_chunks;    // reference chunks (one partial top-k list each) per sequence
  int k3;        // K features of the W3 product (d_ff): the packed W3 rows hold k3 values
  int kdh;       // elements per delta_h row: 2*d_ff bf16 (hi and lo), d_ff fp32
  int n_sink;
  double alpha;
  bool ref_fp8;           // references kept as FP8 E4M3 (compact store [B][nref][C])
  const Schedule* sched;  // host copy of the schedule (planning the distance items)
};

// Byte offsets of the workspace regions (each 256-byte aligned).
struct Workspace {
  size_t wp, w3p, ysq, refs, proj, part, dh, rpos, nrp, tab,
      selj,   // [B*nr][kl] chosen reference indices of each non-reference token, -1 pads
      total;
};

Shape make_shape(int B, int T, int N, int D, int d_ff, int d_c, int k, int g, int b, int s,
                 bool bf16, double alpha, int n_sink, bool ref_fp8);
// Device schedule tables in the workspace: reference positions, non-reference
// positions, and per position t: ~j for the j-th reference, else the
// non-reference index q.
hipError_t launch_schedule(const Shape& sh, char* ws, const Workspace& L, hipStream_t st);
// The reference positions alone, rpos[nref], copied from the host schedule
// through kernel arguments (no host buffer).
hipError_t launch_ref_positions(const Shape& sh, int* rpos, hipStream_t st);
// FP8 reference store [B][nref][C] of the prefix kv.
hipError_t launch_store_refs(const Shape& sh, const void* kv, uint8_t* store, hipStream_t st);
Workspace plan_workspace(const Shape& sh);

// Each launcher enqueues on `st` and returns hipGetLastError().
// Set-up of an encode in one launch (after the positions of a growing
// schedule): weight repacking (skipped when w1 is null), schedule tables,
// compact reference rows and their norms, and the reference tokens'
// ref_idx rows and zero records (records skipped when codes is null).
hipError_t launch_setup(const Shape& sh, const void* w1, const void* w2, const void* w3,
                        const void* kv, char* ws, const Workspace& L, int32_t* ref_idx,
                        uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z,
                        hipStream_t st);
// The distance scan; with wp (the packed [W1|W2]) non-null, the same launch
// also writes the reference projection P = R[W1|W2] (ws + L.proj).
hipError_t launch_dist(const Shape& sh, const void* kv, char* ws, const Workspace& L,
                       const char* wp, hipStream_t st);
hipError_t launch_merge(const Shape& sh, int32_t* ref_idx, char* ws, const Workspace& L,
                        hipStream_t st);
// The contractions read the packed weights at wp ([2 d_ff][C], W1 and W2
// columns interleaved in blocks of 32) and w3p ([d_c][d_ff]): in the
// workspace (packed by the set-up) or in a caller's pre-packed buffer.
hipError_t launch_swiglu(const Shape& sh, const void* kv, char* ws,
                         const Workspace& L, const char* wp, hipStream_t st);
// W3 product fused with the quantiser; writes the records of non-reference tokens.
hipError_t launch_w3_quant(const Shape& sh, char* ws, const Workspace& L, const char* w3p,
                           uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z,
                           hipStream_t st);
// A pre-packed weight buffer: the same two operands the set-up writes into
// the workspace, at byte offsets wp and w3p.
struct PackedLayout {
  size_t wp, w3p, total;
};
PackedLayout plan_packed(const Shape& sh);
hipError_t launch_pack_weights(const Shape& sh, const void* w1, const void* w2, const void* w3,
                               char* packed, hipStream_t st);
// Quantise rows of z [rows][d_c] one to one into records (stepwise export).
hipError_t launch_quantize(const float* z, int64_t rows, int d_c, int g, int b, uint8_t* codes,
                           uint16_t* scale, uint16_t* zmin, hipStream_t st);
hipError_t launch_gather(const uint8_t* codes, const uint16_t* scale, const uint16_t* zmin,
                         const int32_t* idx, int64_t n_idx, int64_t total_rows, int d_c, int g,
                         int b, void* out, bool out_bf16, hipStream_t st);

// Restore ([RKV] §2.5): workspace of the decoder product for n_idx rows.
struct RestoreWorkspace {
  int kr;               // K latents of the decoder product (d_c)
  bool tables;          // schedule tables present (FP8 store of a dynamic schedule)
  size_t wdp, zt,
      rinfo,            // [n_idx][kl + 4] per selected row: its kl stored reference rows
                        // (-1 none), 1/count (float bits), its position (-1 invalid)
      rpos, nrp, tab, total;
};
RestoreWorkspace plan_restore(const Shape& sh, int64_t n_idx);
// The decoder weight packed for the restore's matrix cores ([C][d_c] rows):
// its bytes, and the launch that writes it from wd [d_c][C].
size_t packed_decoder_bytes(const Shape& sh);
hipError_t launch_pack_decoder(const Shape& sh, const void* wd, char* wdp, hipStream_t st);
// The restore from the packed decoder weight wdp (in the workspace at L.wdp,
// packed by rkv_restore, or a caller's buffer from rkv_pack_decoder).
hipError_t launch_restore(const Shape& sh, int N, int D, const uint8_t* codes,
                          const uint16_t* scale, const uint16_t* zmin, const int32_t* ref_idx,
                          const void* kv, const char* wdp, const int32_t* idx, int n_idx,
                          float theta, void* out, bool out_bf16, char* ws,
                          const RestoreWorkspace& L, hipStream_t st);

// Append ([RKV] §2.7 decode step 4): one new token per sequence.
struct AppendWorkspace {
  int n_lists;          // distance workgroups (partial lists) per sequence
  int n_split;          // slices of the C rows of W1 | W2, one workgroup each
  int rb;               // appended tokens per projection workgroup (2 or 4)
  size_t rpos, part, ph, act, total;
};
AppendWorkspace plan_append(const Shape& sh);
// Size of the fixed device scratch the allocation-free append works in.
constexpr size_t kAppendScratchBytes = size_t(4) << 20;
// Device address of that scratch on the current device (looked up once per
// device, then cached); no allocation.
hipError_t append_scratch(char** ptr);
hipError_t launch_append(const Shape& sh, void* kv, const void* kv_new, const int32_t* pos,
                         const void* w1, const void* w2, const void* w3, int32_t* ref_idx,
                         uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z, char* ws,
                         const AppendWorkspace& L, hipStream_t st);
// The append with reference projections: P[b][j] = r_j [W1 | W2] kept with
// the cache (rkv_project_refs fills it, the append extends it).  Its
// workspace (ph holds the tokens' partial projections) also serves
// rkv_project_refs.
AppendWorkspace plan_append_proj(const Shape& sh);
AppendWorkspace plan_project_refs(const Shape& sh);
struct SchedView;  // rkv_device.h
// rkv_project_refs on the matrix cores (bf16 input-precision references):
// the bytes of its packed W1 | W2, 0 where it does not apply (fp32, FP8
// store: the vector-ALU kernel), and the launch (packing, then the tiles).
size_t ref_proj_pack_bytes(const Shape& sh);
hipError_t launch_ref_proj_mfma(const Shape& sh, const void* kv, const void* w1, const void* w2,
                                const SchedView& sv, char* wp, float* proj, hipStream_t st);
hipError_t launch_project_refs(const Shape& sh, const void* kv, const void* w1, const void* w2,
                               float* ref_proj, char* ws, const AppendWorkspace& L,
                               hipStream_t st);
hipError_t launch_append_proj(const Shape& sh, void* kv, float* ref_proj, const void* kv_new,
                              const int32_t* pos, const void* w1, const void* w2, const void* w3,
                              int32_t* ref_idx, uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                              float* z, char* ws, const AppendWorkspace& L, hipStream_t st);

}  // namespace rkv
