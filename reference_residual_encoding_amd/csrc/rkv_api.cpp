// librkv C ABI: argument validation, workspace planning, kernel dispatch.
// The operations themselves are documented in include/rkv.h.
#include "rkv.h"

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "rkv_internal.h"

namespace {

thread_local std::string g_last_error;

rkv_status fail(rkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rkv_status ok() {
  g_last_error.clear();
  return RKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// scale / zmin: not read or written in identity mode (b = 16), may be NULL there
#define RKV_NEED_GROUP_PTR(ptr)                                                        \
  do {                                                                                 \
    if (p->b != 16) RKV_NEED_PTR(ptr);                                                 \
  } while (0)

#define RKV_NEED_PTR(ptr)                                                              \
  do {                                                                                 \
    if ((ptr) == nullptr) return fail(RKV_ERR_INVALID_ARG, "%s is NULL", #ptr);        \
    if (!aligned16(ptr)) return fail(RKV_ERR_INVALID_ARG, "%s is not 16-byte aligned", #ptr); \
  } while (0)

// Fields read by the quantiser and the gather.
rkv_status check_record(const rkv_params* p) {
  if (p->d_c <= 0) return fail(RKV_ERR_INVALID_ARG, "d_c must be positive (got %d)", p->d_c);
  if (p->b != 2 && p->b != 4 && p->b != 16)
    return fail(RKV_ERR_INVALID_ARG, "b must be 2, 4 or 16 (identity) (got %d)", p->b);
  if (p->b == 16) {                       // identity: no groups; g is not read
    if (p->d_c % 32 != 0)
      return fail(RKV_ERR_UNSUPPORTED, "d_c must be a multiple of 32 (got %d)", p->d_c);
    return RKV_OK;
  }
  if (p->g <= 0) return fail(RKV_ERR_INVALID_ARG, "g must be positive (got %d)", p->g);
  if (p->g != 8 && p->g != 16 && p->g != 32 && p->g != 64)
    return fail(RKV_ERR_UNSUPPORTED, "g must be 8, 16, 32 or 64 on the GPU path (got %d)", p->g);
  if (p->d_c % 32 != 0)
    return fail(RKV_ERR_UNSUPPORTED, "d_c must be a multiple of 32 (got %d)", p->d_c);
  if (p->d_c % p->g != 0)
    return fail(RKV_ERR_UNSUPPORTED, "g must divide d_c (g=%d, d_c=%d)", p->g, p->d_c);
  return RKV_OK;
}

rkv_status check_params(const rkv_params* p) {
  if (p == nullptr) return fail(RKV_ERR_INVALID_ARG, "params is NULL");
  if (p->B <= 0 || p->T <= 0) return fail(RKV_ERR_INVALID_ARG, "B and T must be positive (B=%d, T=%d)", p->B, p->T);
  if (p->N <= 0 || p->D <= 0) return fail(RKV_ERR_INVALID_ARG, "N and D must be positive (N=%d, D=%d)", p->N, p->D);
  if (p->d_ff <= 0) return fail(RKV_ERR_INVALID_ARG, "d_ff must be positive (got %d)", p->d_ff);
  if (p->k <= 0) return fail(RKV_ERR_INVALID_ARG, "k must be positive (got %d)", p->k);
  if (p->ref_stride <= 0) return fail(RKV_ERR_INVALID_ARG, "ref_stride must be positive (got %d)", p->ref_stride);
  if (p->dtype != RKV_F32 && p->dtype != RKV_BF16) return fail(RKV_ERR_INVALID_ARG, "unknown dtype %d", int(p->dtype));
  rkv_status st = check_record(p);
  if (st != RKV_OK) return st;
  if (p->k > 8) return fail(RKV_ERR_UNSUPPORTED, "k must be at most 8 on the GPU path (got %d)", p->k);
  const long long C = 2LL * p->N * p->D;
  if (C > (1LL << 20)) return fail(RKV_ERR_UNSUPPORTED, "C = 2*N*D too large (%lld)", C);
  if (C % 64 != 0) return fail(RKV_ERR_UNSUPPORTED, "C = 2*N*D must be a multiple of 64 (got %lld)", C);
  if (p->d_ff % 32 != 0) return fail(RKV_ERR_UNSUPPORTED, "d_ff must be a multiple of 32 (got %d)", p->d_ff);
  if (p->d_ff > 65536) return fail(RKV_ERR_UNSUPPORTED, "d_ff must be at most 65536 (got %d)", p->d_ff);
  // (keeps a 256-row tile of the latent operands within a buffer resource)
  if (p->d_c > 65536) return fail(RKV_ERR_UNSUPPORTED, "d_c must be at most 65536 (got %d)", p->d_c);
  if ((long long)p->B * p->T >= (1LL << 31)) return fail(RKV_ERR_UNSUPPORTED, "B*T must be below 2^31");
  if (p->T > (1 << 26)) return fail(RKV_ERR_UNSUPPORTED, "T must be at most 2^26 (got %d)", p->T);
  if ((long long)p->B * p->T * C >= (1LL << 40)) return fail(RKV_ERR_UNSUPPORTED, "B*T*C too large");
  if (!(p->ref_alpha >= 0.0 && p->ref_alpha <= 1.0e6))
    return fail(RKV_ERR_INVALID_ARG, "ref_alpha must be in [0, 1e6] (got %g)", p->ref_alpha);
  if (p->n_sink < 0) return fail(RKV_ERR_INVALID_ARG, "n_sink must be non-negative (got %d)", p->n_sink);
  if (p->ref_format != RKV_REF_INPUT && p->ref_format != RKV_REF_FP8)
    return fail(RKV_ERR_INVALID_ARG, "unknown ref_format %d", int(p->ref_format));
  const long long nref =
      (long long)rkv::schedule_for(p->T, p->ref_stride, p->ref_alpha, p->n_sink).rpos.size();
  if ((long long)p->B * nref * 2 * p->d_ff * 4 >= (1LL << 31))
    return fail(RKV_ERR_UNSUPPORTED, "B*nref*2*d_ff*4 (reference projections) must be below 2^31 bytes");
  return RKV_OK;
}

rkv::Shape shape_of(const rkv_params* p) {
  return rkv::make_shape(p->B, p->T, p->N, p->D, p->d_ff, p->d_c, p->k, p->g, p->b, p->ref_stride,
                         p->dtype == RKV_BF16, p->ref_alpha, p->n_sink,
                         p->ref_format == RKV_REF_FP8);
}

rkv_status device_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(RKV_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

// Stage profiling: HIP event pairs recorded around selected stages.
struct Profiler {
  std::mutex mu;
  uint32_t mask = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[RKV_STAGE_COUNT];
  size_t used[RKV_STAGE_COUNT] = {};
};
Profiler g_prof;

struct StageScope {
  hipEvent_t end = nullptr;
  hipStream_t st;
  StageScope(int stage, hipStream_t s) : st(s) {
    if (!(g_prof.mask & (1u << stage))) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    auto& v = g_prof.ev[stage];
    size_t& n = g_prof.used[stage];
    if (n == v.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      v.emplace_back(a, b);
    }
    if (hipEventRecord(v[n].first, st) != hipSuccess) return;
    end = v[n].second;
    ++n;
  }
  ~StageScope() {
    if (end) (void)hipEventRecord(end, st);
  }
};

// One stage on `stream`, with its profiling events; a failed launch returns.
#define RKV_STAGE(stage, call, name)                          \
  do {                                                        \
    StageScope scope_(stage, stream);                         \
    if ((e = (call)) != hipSuccess) return device_status(e, name); \
  } while (0)

// The encode after its set-up launch: the distance scan (whose launch also
// computes the reference projection from the packed weights wp), the top-k
// merge, the SwiGLU product, and W3 with the quantiser.
rkv_status encode_after_setup(const rkv::Shape& sh, const void* kv, char* ws,
                              const rkv::Workspace& L, const char* wp, const char* w3p,
                              int32_t* ref_idx, uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                              float* z, hipStream_t stream) {
  hipError_t e;
  RKV_STAGE(RKV_STAGE_DIST, rkv::launch_dist(sh, kv, ws, L, wp, stream), "dist");
  RKV_STAGE(RKV_STAGE_MERGE, rkv::launch_merge(sh, ref_idx, ws, L, stream), "merge");
  if (sh.nr > 0) {
    RKV_STAGE(RKV_STAGE_SWIGLU, rkv::launch_swiglu(sh, kv, ws, L, wp, stream), "swiglu");
    RKV_STAGE(RKV_STAGE_W3, rkv::launch_w3_quant(sh, ws, L, w3p, codes, scale, zmin, z, stream),
              "w3");
  }
  return ok();
}

}  // namespace

extern "C" {

rkv_status rkv_profile_begin(uint32_t stage_mask) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.mask = stage_mask & ((1u << RKV_STAGE_COUNT) - 1);
  for (auto& u : g_prof.used) u = 0;
  return ok();
}

rkv_status rkv_profile_read(int32_t stage, double* total_ms, int64_t* launches) {
  if (stage < 0 || stage >= RKV_STAGE_COUNT) return fail(RKV_ERR_INVALID_ARG, "bad stage %d", stage);
  if (!total_ms || !launches) return fail(RKV_ERR_INVALID_ARG, "output pointer is NULL");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  double sum = 0.0;
  for (size_t i = 0; i < g_prof.used[stage]; ++i) {
    auto& pr = g_prof.ev[stage][i];
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return device_status(e, "profile");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return device_status(e, "profile");
    sum += ms;
  }
  *total_ms = sum;
  *launches = int64_t(g_prof.used[stage]);
  return ok();
}

int rkv_abi_version(void) { return RKV_ABI_VERSION; }

const char* rkv_status_str(rkv_status s) {
  switch (s) {
    case RKV_OK: return "RKV_OK";
    case RKV_ERR_INVALID_ARG: return "RKV_ERR_INVALID_ARG";
    case RKV_ERR_UNSUPPORTED: return "RKV_ERR_UNSUPPORTED";
    case RKV_ERR_WORKSPACE: return "RKV_ERR_WORKSPACE";
    case RKV_ERR_DEVICE: return "RKV_ERR_DEVICE";
  }
  return "RKV_ERR_UNKNOWN";
}

const char* rkv_last_error(void) { return g_last_error.c_str(); }

size_t rkv_encode_workspace_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::plan_workspace(shape_of(p)).total;
}

rkv_status rkv_encode(const rkv_params* p, const void* kv, const void* w1, const void* w2,
                      const void* w3, int32_t* ref_idx, uint8_t* codes, uint16_t* scale,
                      uint16_t* zmin, float* z, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(w3);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(workspace);
  if (z != nullptr && !aligned16(z)) return fail(RKV_ERR_INVALID_ARG, "z is not 16-byte aligned");
  const rkv::Shape sh = shape_of(p);
  const rkv::Workspace L = rkv::plan_workspace(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_NORMS,
            rkv::launch_setup(sh, w1, w2, w3, kv, ws, L, ref_idx, codes, scale, zmin, z, stream),
            "setup");
  return encode_after_setup(sh, kv, ws, L, ws + L.wp, ws + L.w3p, ref_idx, codes, scale, zmin,
                            z, stream);
}

size_t rkv_packed_weights_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::plan_packed(shape_of(p)).total;
}

rkv_status rkv_pack_weights(const rkv_params* p, const void* w1, const void* w2, const void* w3,
                            void* packed, size_t packed_bytes, hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(w3);
  RKV_NEED_PTR(packed);
  const rkv::Shape sh = shape_of(p);
  const rkv::PackedLayout P = rkv::plan_packed(sh);
  if (packed_bytes < P.total)
    return fail(RKV_ERR_WORKSPACE, "packed buffer has %zu bytes, needs %zu", packed_bytes, P.total);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_PACK,
            rkv::launch_pack_weights(sh, w1, w2, w3, static_cast<char*>(packed), stream), "pack");
  return ok();
}

rkv_status rkv_encode_packed(const rkv_params* p, const void* kv, const void* packed,
                             size_t packed_bytes, int32_t* ref_idx, uint8_t* codes,
                             uint16_t* scale, uint16_t* zmin, float* z, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(packed);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(workspace);
  if (z != nullptr && !aligned16(z)) return fail(RKV_ERR_INVALID_ARG, "z is not 16-byte aligned");
  const rkv::Shape sh = shape_of(p);
  const rkv::PackedLayout P = rkv::plan_packed(sh);
  if (packed_bytes < P.total)
    return fail(RKV_ERR_WORKSPACE, "packed buffer has %zu bytes, needs %zu", packed_bytes, P.total);
  const rkv::Workspace L = rkv::plan_workspace(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  const char* wp = static_cast<const char*>(packed) + P.wp;
  const char* w3p = static_cast<const char*>(packed) + P.w3p;
  hipError_t e;
  // the set-up without the weight repacking (w1 null)
  RKV_STAGE(RKV_STAGE_NORMS,
            rkv::launch_setup(sh, nullptr, nullptr, nullptr, kv, ws, L, ref_idx, codes, scale,
                              zmin, z, stream),
            "setup");
  return encode_after_setup(sh, kv, ws, L, wp, w3p, ref_idx, codes, scale, zmin, z, stream);
}

rkv_status rkv_select(const rkv_params* p, const void* kv, int32_t* ref_idx, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(workspace);
  const rkv::Shape sh = shape_of(p);
  const rkv::Workspace L = rkv::plan_workspace(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_NORMS,
            rkv::launch_setup(sh, nullptr, nullptr, nullptr, kv, ws, L, ref_idx, nullptr, nullptr,
                              nullptr, nullptr, stream),
            "setup");
  RKV_STAGE(RKV_STAGE_DIST, rkv::launch_dist(sh, kv, ws, L, nullptr, stream), "dist");
  RKV_STAGE(RKV_STAGE_MERGE, rkv::launch_merge(sh, ref_idx, ws, L, stream), "merge");
  return ok();
}

rkv_status rkv_quantize(const rkv_params* p, const float* z, int64_t rows, uint8_t* codes,
                        uint16_t* scale, uint16_t* zmin, hipStream_t stream) {
  if (p == nullptr) return fail(RKV_ERR_INVALID_ARG, "params is NULL");
  rkv_status st = check_record(p);
  if (st != RKV_OK) return st;
  if (rows < 0) return fail(RKV_ERR_INVALID_ARG, "rows must be non-negative (got %lld)", (long long)rows);
  if (rows * (long long)p->d_c >= (1LL << 40)) return fail(RKV_ERR_UNSUPPORTED, "rows*d_c too large");
  if (rows == 0) return ok();
  RKV_NEED_PTR(z);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_QUANT,
            rkv::launch_quantize(z, rows, p->d_c, p->g, p->b, codes, scale, zmin, stream),
            "quantize");
  return ok();
}

rkv_status rkv_dequant_gather(const rkv_params* p, const uint8_t* codes, const uint16_t* scale,
                              const uint16_t* zmin, const int32_t* idx, int32_t n_idx, void* out,
                              rkv_dtype out_dtype, hipStream_t stream) {
  if (p == nullptr) return fail(RKV_ERR_INVALID_ARG, "params is NULL");
  rkv_status st = check_record(p);
  if (st != RKV_OK) return st;
  if (p->B <= 0 || p->T <= 0) return fail(RKV_ERR_INVALID_ARG, "B and T must be positive (B=%d, T=%d)", p->B, p->T);
  if (n_idx < 0) return fail(RKV_ERR_INVALID_ARG, "n_idx must be non-negative (got %d)", n_idx);
  if (out_dtype != RKV_F32 && out_dtype != RKV_BF16) return fail(RKV_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (n_idx == 0) return ok();
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(idx);
  RKV_NEED_PTR(out);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_GATHER,
            rkv::launch_gather(codes, scale, zmin, idx, n_idx, int64_t(p->B) * p->T, p->d_c, p->g,
                               p->b, out, out_dtype == RKV_BF16, stream),
            "gather");
  return ok();
}

// Restore shares the encode's parameter checks and needs whole heads per
// 128-column tile (the rotation partner d +- D/2 sits in the same tile).
static rkv_status check_restore(const rkv_params* p, int32_t n_idx) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if (p->D % 16 != 0 || 128 % p->D != 0)
    return fail(RKV_ERR_UNSUPPORTED, "restore needs D in {16, 32, 64, 128} (got %d)", p->D);
  if (n_idx < 0) return fail(RKV_ERR_INVALID_ARG, "n_idx must be non-negative (got %d)", n_idx);
  return RKV_OK;
}

size_t rkv_restore_workspace_bytes(const rkv_params* p, int32_t n_idx) {
  if (check_restore(p, n_idx) != RKV_OK) return 0;
  return rkv::plan_restore(shape_of(p), n_idx).total;
}

// The checks and launches of rkv_restore (is_packed false: wd the unpacked
// weight, packed into the workspace first) and rkv_restore_packed
// (is_packed true: the caller's packed buffer of packed_bytes).
static rkv_status restore_common(const rkv_params* p, const uint8_t* codes, const uint16_t* scale,
                                 const uint16_t* zmin, const int32_t* ref_idx, const void* kv,
                                 bool is_packed, const void* wd, const void* packed, size_t packed_bytes,
                                 const int32_t* idx, int32_t n_idx, float rope_theta, void* out,
                                 rkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  rkv_status st = check_restore(p, n_idx);
  if (st != RKV_OK) return st;
  if (out_dtype != RKV_F32 && out_dtype != RKV_BF16)
    return fail(RKV_ERR_INVALID_ARG, "unknown out_dtype %d", int(out_dtype));
  if (!(rope_theta == rope_theta)) return fail(RKV_ERR_INVALID_ARG, "rope_theta is NaN");
  if (n_idx == 0) return ok();
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(kv);
  if (is_packed) RKV_NEED_PTR(packed); else RKV_NEED_PTR(wd);
  RKV_NEED_PTR(idx);
  RKV_NEED_PTR(out);
  RKV_NEED_PTR(workspace);
  const rkv::Shape sh = shape_of(p);
  const rkv::RestoreWorkspace L = rkv::plan_restore(sh, n_idx);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  if (is_packed && packed_bytes < rkv::packed_decoder_bytes(sh))
    return fail(RKV_ERR_WORKSPACE, "packed decoder has %zu bytes, needs %zu", packed_bytes,
                rkv::packed_decoder_bytes(sh));
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (!is_packed)
    RKV_STAGE(RKV_STAGE_PACK, rkv::launch_pack_decoder(sh, wd, ws + L.wdp, stream), "pack");
  const char* w = is_packed ? static_cast<const char*>(packed) : ws + L.wdp;
  RKV_STAGE(RKV_STAGE_RESTORE,
            rkv::launch_restore(sh, p->N, p->D, codes, scale, zmin, ref_idx, kv, w, idx, n_idx,
                                rope_theta, out, out_dtype == RKV_BF16, ws, L, stream),
            "restore");
  return ok();
}

rkv_status rkv_restore(const rkv_params* p, const uint8_t* codes, const uint16_t* scale,
                       const uint16_t* zmin, const int32_t* ref_idx, const void* kv,
                       const void* wd, const int32_t* idx, int32_t n_idx, float rope_theta,
                       void* out, rkv_dtype out_dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return restore_common(p, codes, scale, zmin, ref_idx, kv, false, wd, nullptr, 0, idx, n_idx,
                        rope_theta, out, out_dtype, workspace, workspace_bytes, stream);
}

size_t rkv_packed_decoder_bytes(const rkv_params* p) {
  if (check_restore(p, 0) != RKV_OK) return 0;
  return rkv::packed_decoder_bytes(shape_of(p));
}

rkv_status rkv_pack_decoder(const rkv_params* p, const void* wd, void* packed,
                            size_t packed_bytes, hipStream_t stream) {
  rkv_status st = check_restore(p, 0);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(wd);
  RKV_NEED_PTR(packed);
  const rkv::Shape sh = shape_of(p);
  if (packed_bytes < rkv::packed_decoder_bytes(sh))
    return fail(RKV_ERR_WORKSPACE, "packed decoder has %zu bytes, needs %zu", packed_bytes,
                rkv::packed_decoder_bytes(sh));
  hipError_t e;
  RKV_STAGE(RKV_STAGE_PACK,
            rkv::launch_pack_decoder(sh, wd, static_cast<char*>(packed), stream), "pack");
  return ok();
}

rkv_status rkv_restore_packed(const rkv_params* p, const uint8_t* codes, const uint16_t* scale,
                              const uint16_t* zmin, const int32_t* ref_idx, const void* kv,
                              const void* packed, size_t packed_bytes, const int32_t* idx,
                              int32_t n_idx, float rope_theta, void* out, rkv_dtype out_dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return restore_common(p, codes, scale, zmin, ref_idx, kv, true, nullptr, packed, packed_bytes,
                        idx, n_idx, rope_theta, out, out_dtype, workspace, workspace_bytes,
                        stream);
}

size_t rkv_append_workspace_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::plan_append(shape_of(p)).total;
}

rkv_status rkv_append(const rkv_params* p, void* kv, const void* kv_new, const int32_t* pos,
                      const void* w1, const void* w2, const void* w3, int32_t* ref_idx,
                      uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(kv_new);
  RKV_NEED_PTR(pos);
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(w3);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(workspace);
  if (z != nullptr && !aligned16(z)) return fail(RKV_ERR_INVALID_ARG, "z is not 16-byte aligned");
  const rkv::Shape sh = shape_of(p);
  const rkv::AppendWorkspace L = rkv::plan_append(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_APPEND,
            rkv::launch_append(sh, kv, kv_new, pos, w1, w2, w3, ref_idx, codes, scale, zmin, z,
                               static_cast<char*>(workspace), L, stream),
            "append");
  return ok();
}

rkv_status rkv_append_noalloc(const rkv_params* p, void* kv, const void* kv_new,
                              const int32_t* pos, const void* w1, const void* w2, const void* w3,
                              int32_t* ref_idx, uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                              float* z, hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(kv_new);
  RKV_NEED_PTR(pos);
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(w3);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  if (z != nullptr && !aligned16(z)) return fail(RKV_ERR_INVALID_ARG, "z is not 16-byte aligned");
  const rkv::Shape sh = shape_of(p);
  const rkv::AppendWorkspace L = rkv::plan_append(sh);
  if (L.total > rkv::kAppendScratchBytes)
    return fail(RKV_ERR_WORKSPACE,
                "rkv_append_noalloc needs %zu bytes of scratch, more than its fixed %zu; "
                "use rkv_append with a workspace",
                L.total, rkv::kAppendScratchBytes);
  char* ws = nullptr;
  hipError_t e = rkv::append_scratch(&ws);
  if (e != hipSuccess)
    return fail(RKV_ERR_DEVICE, "scratch address: %s", hipGetErrorString(e));
  RKV_STAGE(RKV_STAGE_APPEND,
            rkv::launch_append(sh, kv, kv_new, pos, w1, w2, w3, ref_idx, codes, scale, zmin, z,
                               ws, L, stream),
            "append");
  return ok();
}

size_t rkv_ref_proj_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  const rkv::Shape sh = shape_of(p);
  return size_t(sh.B) * sh.nref * 2 * sh.d_ff * 4;
}

size_t rkv_append_proj_workspace_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::plan_append_proj(shape_of(p)).total;
}

size_t rkv_project_refs_workspace_bytes(const rkv_params* p) {
  if (check_params(p) != RKV_OK) return 0;
  return rkv::plan_project_refs(shape_of(p)).total;
}

rkv_status rkv_project_refs(const rkv_params* p, const void* kv, const void* w1, const void* w2,
                            float* ref_proj, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(ref_proj);
  RKV_NEED_PTR(workspace);
  const rkv::Shape sh = shape_of(p);
  const rkv::AppendWorkspace L = rkv::plan_project_refs(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_APPEND,
            rkv::launch_project_refs(sh, kv, w1, w2, ref_proj, static_cast<char*>(workspace), L,
                                     stream),
            "project_refs");
  return ok();
}

rkv_status rkv_append_proj(const rkv_params* p, void* kv, float* ref_proj, const void* kv_new,
                           const int32_t* pos, const void* w1, const void* w2, const void* w3,
                           int32_t* ref_idx, uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                           float* z, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(ref_proj);
  RKV_NEED_PTR(kv_new);
  RKV_NEED_PTR(pos);
  RKV_NEED_PTR(w1);
  RKV_NEED_PTR(w2);
  RKV_NEED_PTR(w3);
  RKV_NEED_PTR(ref_idx);
  RKV_NEED_PTR(codes);
  RKV_NEED_GROUP_PTR(scale);
  RKV_NEED_GROUP_PTR(zmin);
  RKV_NEED_PTR(workspace);
  if (z != nullptr && !aligned16(z)) return fail(RKV_ERR_INVALID_ARG, "z is not 16-byte aligned");
  if (!aligned16(ref_proj)) return fail(RKV_ERR_INVALID_ARG, "ref_proj is not 16-byte aligned");
  const rkv::Shape sh = shape_of(p);
  const rkv::AppendWorkspace L = rkv::plan_append_proj(sh);
  if (workspace_bytes < L.total)
    return fail(RKV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_APPEND,
            rkv::launch_append_proj(sh, kv, ref_proj, kv_new, pos, w1, w2, w3, ref_idx, codes,
                                    scale, zmin, z, static_cast<char*>(workspace), L, stream),
            "append_proj");
  return ok();
}

rkv_status rkv_store_refs(const rkv_params* p, const void* kv, uint8_t* ref_store,
                          hipStream_t stream) {
  rkv_status st = check_params(p);
  if (st != RKV_OK) return st;
  if (p->ref_format != RKV_REF_FP8)
    return fail(RKV_ERR_INVALID_ARG, "rkv_store_refs needs ref_format RKV_REF_FP8");
  RKV_NEED_PTR(kv);
  RKV_NEED_PTR(ref_store);
  const rkv::Shape sh = shape_of(p);
  hipError_t e;
  RKV_STAGE(RKV_STAGE_STORE, rkv::launch_store_refs(sh, kv, ref_store, stream), "store");
  return ok();
}

int32_t rkv_reference_positions(const rkv_params* p, int32_t* rpos, int32_t cap) {
  if (p == nullptr) { fail(RKV_ERR_INVALID_ARG, "params is NULL"); return -1; }
  if (p->T <= 0 || p->T > (1 << 26)) { fail(RKV_ERR_INVALID_ARG, "T must be in [1, 2^26] (got %d)", p->T); return -1; }
  if (p->ref_stride <= 0) { fail(RKV_ERR_INVALID_ARG, "ref_stride must be positive (got %d)", p->ref_stride); return -1; }
  if (!(p->ref_alpha >= 0.0 && p->ref_alpha <= 1.0e6)) { fail(RKV_ERR_INVALID_ARG, "ref_alpha must be in [0, 1e6]"); return -1; }
  if (p->n_sink < 0) { fail(RKV_ERR_INVALID_ARG, "n_sink must be non-negative (got %d)", p->n_sink); return -1; }
  if (cap < 0 || (cap > 0 && rpos == nullptr)) { fail(RKV_ERR_INVALID_ARG, "rpos is NULL or cap negative"); return -1; }
  const auto& sc = rkv::schedule_for(p->T, p->ref_stride, p->ref_alpha, p->n_sink);
  const int32_t n = int32_t(sc.rpos.size());
  for (int32_t i = 0; i < n && i < cap; ++i) rpos[i] = sc.rpos[size_t(i)];
  ok();
  return n;
}

}  // extern "C"
