/*
 * rkv.h - C ABI of librkv, the ResidualKV cache-write path for AMD MI355X
 * (gfx950).
 *
 * Source of the method: the ResidualKV reading notes, "ResidualKV：基于参考向量
 * 与残差的 KV Cache 压缩" (notes on arXiv 2602.08005v2), cited as [RKV] with the
 * notes' own section numbers.  Argument names follow the notes' symbol table
 * ([RKV] §2.1): B sequences of T tokens, N KV heads of dimension D, joint
 * vector width C = 2*d_k = 2*N*D, compressor width d_ff, latent width d_c,
 * k neighbours, quantiser group g and bit width b ([RKV] §2.4), reference
 * stride s ([RKV] §2.6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller (HBM of
 *    the device that is current on the calling thread), 16-byte aligned.
 *    The library never allocates, frees or synchronises; all work is
 *    enqueued on `stream` and the call returns before it finishes.  Results
 *    are valid once the stream is synchronised.  Two calls may run
 *    concurrently on different streams if each has its own workspace.
 *  - Every argument check runs on the host before anything is enqueued.  On
 *    failure nothing is enqueued, the status is returned and
 *    rkv_last_error() describes it (thread-local text).  A launch failure
 *    reported by the HIP runtime returns RKV_ERR_DEVICE; a fault inside a
 *    kernel surfaces at the caller's next synchronisation.
 *  - Results are bitwise deterministic: no atomics decide any value.
 *  - Token layout: kv[b][t][c] with c in [0, C): the N key heads (pre-RoPE)
 *    then the N value heads, D coordinates each ([RKV] §2.1: K and V of all
 *    heads flattened into one joint vector).
 *  - Reference schedule ([RKV] §2.6): positions t < n_sink (sink tokens)
 *    are references; then p_0 = n_sink and p_{m+1} = p_m + s +
 *    floor(ref_alpha * (p_m - n_sink)) (the floor of the double product).
 *    With ref_alpha = 0 and n_sink = 0 the references are t % s == 0 (fixed
 *    stride).  The candidate pool of a non-reference token t holds the
 *    references at positions j < t of the same sequence; k_t = min(k, pool
 *    size) ([RKV] §2.1).  Position 0 is always a reference.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_ABI_VERSION 8

typedef enum {
  RKV_OK = 0,
  RKV_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or field     */
  RKV_ERR_UNSUPPORTED = 2, /* valid for the method, not for this GPU path     */
  RKV_ERR_WORKSPACE = 3,   /* workspace smaller than *_workspace_bytes()      */
  RKV_ERR_DEVICE = 4       /* the HIP runtime reported an error               */
} rkv_status;

typedef enum { RKV_F32 = 0, RKV_BF16 = 1 } rkv_dtype;

/* How the cache keeps its references ([RKV] §2.4 last paragraph: stored
 * as they are, in FP8 in deployment; §2.5: encoder and decoder use them as
 * stored).
 *   RKV_REF_INPUT: at input precision, the rows kv[b][t] at reference
 *                  positions t (p->dtype).
 *   RKV_REF_FP8:   as OCP FP8 E4M3 bytes (bias 7, 3 mantissa bits, largest
 *                  finite 448; round to nearest even, saturating at +-448,
 *                  no scale factor) in a compact store ref_store[b][j][C],
 *                  j the index of the reference in the schedule.  The
 *                  encode computes with the FP8 values of kv's reference
 *                  rows; rkv_store_refs writes the store; rkv_restore and
 *                  rkv_append read (and append writes) the store. */
typedef enum { RKV_REF_INPUT = 0, RKV_REF_FP8 = 1 } rkv_ref_format;

typedef struct {
  int32_t B, T;       /* sequences; tokens per sequence                        */
  int32_t N, D;       /* KV heads; head dimension.  C = 2*N*D                  */
  int32_t d_ff, d_c;  /* compressor width; latent width                        */
  int32_t k;          /* neighbours per token, 1..8 ([RKV] §2.2 uses 4)        */
  int32_t g, b;       /* quantiser group size (8,16,32,64); bits 2 or 4, or 16:
                         quantisation off ([RKV] §2.4: Q is the identity), the
                         latent stored as fp16 and no group numbers (scale,
                         zmin neither read nor written, may be NULL; g unused) */
  int32_t ref_stride; /* s >= 1 (s0, the initial stride, of the schedule)      */
  rkv_dtype dtype;    /* element type of kv, w1, w2, w3                        */
  int32_t n_sink;     /* sink tokens (positions < n_sink), stored as references */
  double ref_alpha;   /* schedule growth alpha >= 0 ([RKV] §2.6); 0: fixed     */
  int32_t ref_format; /* rkv_ref_format of the stored references             */
} rkv_params;

/* GPU-path limits (RKV_ERR_UNSUPPORTED otherwise): C % 64 == 0,
 * d_ff % 32 == 0, d_ff <= 65536, d_c % 32 == 0, d_c <= 65536, d_c % g == 0, B*T < 2^31,
 * T <= 2^26, B*nref*2*d_ff*4 < 2^31 with nref the references per sequence
 * (the reference projections).
 *
 * Environment: RKV_DMA_GLOBAL=1 (read at every call) makes the contractions
 * over kv rows copy their operands to LDS with 64-bit lane addresses instead
 * of 32-bit offsets from a buffer resource.  Results are bit-identical; the
 * library takes that form by itself where a tile's kv rows span 2 GB or
 * more.  RKV_SWIGLU_ORDER=row or =col (read at every call) forces the order
 * in which the SwiGLU product visits its tiles (row tile fastest, or column
 * tile fastest, which the library takes by itself once B*T*C*esize exceeds
 * 192 MiB); results are bit-identical.  RKV_DIST_TILE=wide, =narrow or
 * =short (read at every call) forces the distance launch's tiling (8 waves
 * on 256 tokens; 4 waves on 128 tokens two workgroups to a CU, which the
 * library takes for bf16 where C <= 1024; the same on chunks of 128
 * references, which it takes where the wide tiles give under two rounds of
 * work items); results are bit-identical, and the workspace size does not
 * depend on the tiling.  RKV_W3_TILE=wide or =narrow
 * likewise forces the tiling of the W3 product with the quantiser (256 x 256,
 * or 128 x 128 two workgroups to a CU, which the library takes for bf16 where
 * the wide tiles would number fewer than half the CUs).  RKV_RESTORE_TILE=wide
 * or =narrow likewise forces the tiling of rkv_restore's decoder product
 * (256 x 256, or 128 x 128 two workgroups to a CU, which the library takes
 * for bf16 where the wide tiles would fill at most half the CUs). */

/* Bytes of device workspace rkv_encode / rkv_select need for *p (0 if *p is
 * invalid).  The workspace holds repacked weights, reference projections,
 * partial neighbour lists, the SwiGLU difference and the latent; its
 * contents are private and need not be initialised. */
size_t rkv_encode_workspace_bytes(const rkv_params* p);

/* Encode a whole prefix of B sequences into the ResidualKV cache format.
 *
 * For every non-reference token t ([RKV] §2.2-§2.4):
 *   R_t   = the k_t references nearest to kv_t in squared L2 over all C
 *           coordinates (ties: smaller position first)   [RKV] §2.2 eq. 1
 *   m_t   = mean of kv_j over j in R_t                   [RKV] §2.2 eq. 2
 *   f_c(x)= (Swish(x W1) * (x W2)) W3, Swish = SiLU      [RKV] §2.3
 *   z_t   = f_c(kv_t) - f_c(m_t)                         [RKV] §2.3 boxed eq.
 *   per group of g consecutive latent coordinates: Delta = (max-min)/(2^b-1),
 *   Delta_h = fp16(Delta), m_h = fp16(min),
 *   q = clamp(rint((z - m_h)/Delta_h), 0, 2^b-1), q = 0 when Delta_h == 0
 *                                                        [RKV] §2.4
 * Reference tokens are stored as they are by the caller ([RKV] §2.4): their
 * ref_idx row is all -1 and their record (codes, scale, zmin, z) is zero.
 *
 * Inputs:  kv [B][T][C]; w1, w2 [C][d_ff]; w3 [d_ff][d_c]; row-major, the
 *          element type p->dtype; used as x*W (row vector times matrix).
 * Outputs: ref_idx [B][T][k] int32: chosen reference positions within the
 *                  sequence, ascending; -1 pads when k_t < k.
 *          codes   [B][T][d_c*b/8]: packed little-endian inside a byte
 *                  (coordinate (8/b)*j + r in bits [r*b, (r+1)*b) of byte j).
 *          scale   [B][T][d_c/g]: fp16 bits of Delta_h.
 *          zmin    [B][T][d_c/g]: fp16 bits of m_h.
 *          z       optional [B][T][d_c] float latent (NULL: not written).
 * workspace: at least rkv_encode_workspace_bytes(p) bytes of device memory.
 * Arithmetic: bf16 inputs are multiplied exactly and accumulated in fp32 on
 * the matrix cores; the quantiser works in fp32. */
rkv_status rkv_encode(const rkv_params* p, const void* kv, const void* w1,
                      const void* w2, const void* w3, int32_t* ref_idx,
                      uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                      float* z, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Pre-packed compressor weights.  The compressor f_c's weights W1, W2, W3
 * are fixed once the codec is trained ([RKV] §2.3; §2.5: every token is
 * compressed once, when it is written), so a caller can lay them out once
 * in the operand form the encode's matrix-core products read, instead of
 * rkv_encode repacking them at every call:
 *   rkv_packed_weights_bytes(p): bytes of that buffer for p's C, d_ff, d_c
 *     and dtype (0 if *p is invalid);
 *   rkv_pack_weights: writes it from w1, w2 [C][d_ff] and w3 [d_ff][d_c]
 *     (layouts as rkv_encode; `packed` is caller-owned device memory of at
 *     least rkv_packed_weights_bytes(p) bytes; its layout is private);
 *   rkv_encode_packed: exactly rkv_encode (same outputs, bit for bit, and
 *     the same workspace size) with the weights taken from `packed`.
 * The packed buffer depends only on the weights, C, d_ff, d_c and dtype; it
 * may be shared by any number of calls, including concurrent ones. */
size_t rkv_packed_weights_bytes(const rkv_params* p);
rkv_status rkv_pack_weights(const rkv_params* p, const void* w1, const void* w2,
                            const void* w3, void* packed, size_t packed_bytes,
                            hipStream_t stream);
rkv_status rkv_encode_packed(const rkv_params* p, const void* kv,
                             const void* packed, size_t packed_bytes,
                             int32_t* ref_idx, uint8_t* codes, uint16_t* scale,
                             uint16_t* zmin, float* z, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Selective dequantisation: out[i][:] = q * Delta_h + m_h (one fp32 FMA per
 * coordinate) for the record of flat token idx[i] = b*T + t
 * ([RKV] §2.4 third eq.; §2.7 decode step 3: only selected tokens are
 * decompressed, each from its own record).  Indices may repeat and come in
 * any order; an index outside [0, B*T) yields a row of NaN.  Reference
 * tokens decode to zeros.
 * out: [n_idx][d_c], float (RKV_F32) or bf16 rounded to nearest even
 * (RKV_BF16).  n_idx == 0 is a no-op.  Only p->B, T, d_c, g, b are read. */
rkv_status rkv_dequant_gather(const rkv_params* p, const uint8_t* codes,
                              const uint16_t* scale, const uint16_t* zmin,
                              const int32_t* idx, int32_t n_idx, void* out,
                              rkv_dtype out_dtype, hipStream_t stream);

/* Stepwise export of the quantiser ([RKV] §2.4) alone: quantise `rows`
 * latent rows z [rows][d_c] (float) into codes/scale/zmin laid out as in
 * rkv_encode.  Only p->d_c, g, b are read. */
rkv_status rkv_quantize(const rkv_params* p, const float* z, int64_t rows,
                        uint8_t* codes, uint16_t* scale, uint16_t* zmin,
                        hipStream_t stream);

/* Stepwise export of retrieval ([RKV] §2.2 eq. 1) alone: writes ref_idx as
 * rkv_encode does.  Needs the same workspace size as rkv_encode. */
rkv_status rkv_select(const rkv_params* p, const void* kv, int32_t* ref_idx,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Read side: restore the K|V rows of selected tokens ([RKV] §2.5 boxed eq.;
 * §2.7 decode step 3; §2.1 note on rotating restored keys).
 *
 * For each idx[i] = b*T + t:
 *   non-reference t:  KV^ = z~ W_d + mean of kv_j over the token's ref_idx
 *                     row (j >= 0), z~ = q * Delta_h + m_h of its record
 *                     (fmaf, as rkv_dequant_gather), W_d bias-free
 *   reference t:      KV^ = kv_t (references are stored as they are)
 *   K = KV^[0, N*D) is then rotated at position t when rope_theta > 0:
 *   coordinate d and d + D/2 of a head form pair i = d, turned by the angle
 *   t * rope_theta^(-2i/D) ("rotate half"; angles reduced in fp64, sin/cos
 *   in fp32); V = KV^[N*D, C) as is.  rope_theta <= 0 leaves K unrotated.
 * Inputs:  codes, scale, zmin, ref_idx as rkv_encode wrote them ([B][T]...);
 *          kv: the stored references: with RKV_REF_INPUT kv [B][T][C] in
 *          p->dtype (only rows at reference positions are read), with
 *          RKV_REF_FP8 the store [B][n_ref][C] of E4M3 bytes;
 *          wd [d_c][C] in p->dtype, used as z * W_d; idx [n_idx] int32, any
 *          order, duplicates allowed.
 * Output:  out [n_idx][C], float (RKV_F32) or bf16 rounded to nearest even
 *          (RKV_BF16); an index outside [0, B*T) yields a row of NaN.
 * workspace: at least rkv_restore_workspace_bytes(p, n_idx) bytes.
 * Arithmetic: z~ enters the bf16 matrix cores as a (hi, lo) bf16 pair (fp32
 * inputs use the fp32 matrix cores); products accumulate in fp32.
 * GPU-path limit (RKV_ERR_UNSUPPORTED otherwise): D in {16, 32, 64, 128}. */
size_t rkv_restore_workspace_bytes(const rkv_params* p, int32_t n_idx);
rkv_status rkv_restore(const rkv_params* p, const uint8_t* codes,
                       const uint16_t* scale, const uint16_t* zmin,
                       const int32_t* ref_idx, const void* kv, const void* wd,
                       const int32_t* idx, int32_t n_idx, float rope_theta,
                       void* out, rkv_dtype out_dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* The restore with a pre-packed decoder weight ([RKV] §2.5: W_d is fixed,
 * so the layout the matrix cores read need not be rebuilt at every call):
 *   rkv_packed_decoder_bytes(p): bytes of that buffer for p's C, d_c and
 *     dtype (0 for invalid p);
 *   rkv_pack_decoder: writes it from wd [d_c][C] in p->dtype (packed: a
 *     caller-owned device buffer of at least rkv_packed_decoder_bytes(p)
 *     bytes, 16-byte aligned; its layout is private);
 *   rkv_restore_packed: exactly rkv_restore (the same outputs, bit for
 *     bit) with the packed buffer in place of wd; its workspace is
 *     rkv_restore_workspace_bytes(p, n_idx) as well.
 * Errors as rkv_restore, and RKV_ERR_WORKSPACE when packed_bytes is short.
 * The buffer stays valid for any p with the same C, d_c and dtype. */
size_t rkv_packed_decoder_bytes(const rkv_params* p);
rkv_status rkv_pack_decoder(const rkv_params* p, const void* wd, void* packed,
                            size_t packed_bytes, hipStream_t stream);
rkv_status rkv_restore_packed(const rkv_params* p, const uint8_t* codes,
                              const uint16_t* scale, const uint16_t* zmin,
                              const int32_t* ref_idx, const void* kv,
                              const void* packed, size_t packed_bytes,
                              const int32_t* idx, int32_t n_idx, float rope_theta,
                              void* out, rkv_dtype out_dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Decode-time append ([RKV] §2.7 decode step 4): one new token per
 * sequence enters the cache.  For sequence b the new token sits at position
 * t = pos[b]:
 *   reference t (the schedule above):  kv[b][t] = kv_new[b] (stored as it
 *       is), its ref_idx row all -1 and its record zero;
 *   non-reference t:  encoded exactly as rkv_encode encodes position t, with
 *       the pool read from the cache: the references of sequence b at
 *       positions j < t, rows kv[b][j] ([RKV] §2.2-§2.4); its ref_idx row
 *       and record (and z) are written at b*T + t;
 *   t outside [0, T):  sequence b is left untouched (nothing is written).
 * Only reference rows of kv are read, and only the row of a sequence whose
 * new token is a reference is written; the other rows of kv may hold
 * anything.  Records of other positions are not touched.  Positions of
 * different sequences are independent (continuous batching).
 * Inputs:  kv (in/out), the cache's stored references: with RKV_REF_INPUT
 *          [B][T][C] in p->dtype, rows at positions; with RKV_REF_FP8 the
 *          store [B][n_ref][C] of E4M3 bytes, row j the j-th reference (a
 *          new reference is written there as its E4M3 bytes);
 *          kv_new [B][C], p->dtype, the new tokens (pre-RoPE K | V);
 *          pos [B] int32, device memory; w1, w2, w3 as in rkv_encode.
 * Outputs: ref_idx, codes, scale, zmin, z (optional) laid out as in
 *          rkv_encode, one row per appended token.
 * workspace: at least rkv_append_workspace_bytes(p) bytes (its contents are
 *          private and need not be initialised).
 * Arithmetic: fp32 on the vector ALUs from the stored values: distances by
 * direct differences, the mean in fp32, the products x W1, x W2, m W1,
 * m W2 and delta_h W3 in fp32; the quantiser as in rkv_encode. */
size_t rkv_append_workspace_bytes(const rkv_params* p);
rkv_status rkv_append(const rkv_params* p, void* kv, const void* kv_new,
                      const int32_t* pos, const void* w1, const void* w2,
                      const void* w3, int32_t* ref_idx, uint8_t* codes,
                      uint16_t* scale, uint16_t* zmin, float* z,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* rkv_append without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics, outputs
 * and kernels as rkv_append; the workspace is a fixed 4 MiB array of device
 * memory inside the library (one copy per GPU, loaded with the library and
 * held until the process ends; its address is looked up on the first call
 * on each device).  Nothing is allocated or freed and no allocating routine
 * is called.  Returns RKV_ERR_WORKSPACE, with nothing enqueued, when the
 * call needs more than 4 MiB (rkv_append_workspace_bytes(p) > 4 MiB; at
 * C = 2048, d_ff = 1024 with 2,048 references per sequence every B that
 * rkv_params allows fits: 82 KB at B = 1, 1.6 MB at B = 64): use rkv_append
 * there.  Every call on a GPU shares that GPU's array, so calls that
 * overlap on one GPU (on different streams, or from different threads) race
 * and give undefined results; serialise them on one stream.  The array keeps
 * the last call's contents; nothing in it needs to start at zero. */
rkv_status rkv_append_noalloc(const rkv_params* p, void* kv, const void* kv_new,
                              const int32_t* pos, const void* w1, const void* w2,
                              const void* w3, int32_t* ref_idx, uint8_t* codes,
                              uint16_t* scale, uint16_t* zmin, float* z,
                              hipStream_t stream);

/* Reference projections kept with the cache: ref_proj[b][j][o] =
 * r_j [W1 | W2][o], o < 2 d_ff (the first d_ff outputs through W1, the
 * next through W2), fp32, for the j-th stored reference r_j of sequence b
 * (its stored values: input precision, or the E4M3 values of an FP8
 * store).  The first layer of f_c is linear, so the projection of the
 * chosen references' mean is the mean of their projections ([RKV] §2.2 mean
 * eq., §2.3 f_c): rkv_append_proj reads k_t rows of it instead of
 * projecting the mean through W1 and W2.  rkv_ref_proj_bytes(p) = B *
 * n_ref * 2 * d_ff * 4 (n_ref = rkv_reference_positions(p, NULL, 0)).
 *
 * rkv_project_refs fills every row from the cache kv (laid out as for
 * rkv_append; a row whose reference is not stored yet gets whatever its
 * kv row holds projected); w1, w2 as in rkv_encode.  workspace: at least
 * rkv_project_refs_workspace_bytes(p) bytes (private, need not be
 * initialised).  Arithmetic: with bf16 references kept at input precision,
 * the encode's projection tiles on the matrix cores (bf16 products, fp32
 * sums); otherwise fp32 on the vector ALUs, each output summed over C in
 * chunks of 512 rows. */
size_t rkv_ref_proj_bytes(const rkv_params* p);
size_t rkv_project_refs_workspace_bytes(const rkv_params* p);
size_t rkv_append_proj_workspace_bytes(const rkv_params* p);
rkv_status rkv_project_refs(const rkv_params* p, const void* kv, const void* w1,
                            const void* w2, float* ref_proj, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* rkv_append with the cache's reference projections ref_proj (above): the
 * same outputs and semantics as rkv_append, and, for a sequence whose new
 * token is a reference, ref_proj[b][j] written for it (j its index among
 * the references; from its E4M3 values with an FP8 store).  The mean
 * branch m [W1 | W2] is the mean of the chosen references' rows of
 * ref_proj (summed in ascending position, times 1/k_t) in place of the mean
 * row projected through W1 and W2, so the call runs in two launches: the
 * distances together with x [W1 | W2], then the selection, delta_h, z =
 * delta_h W3 and the quantiser.  Rows of ref_proj of references not in a
 * token's pool are not read.  workspace: at least
 * rkv_append_proj_workspace_bytes(p) bytes (private, need not be
 * initialised).  Results agree with rkv_append within fp32 rounding
 * (the projections are summed in another order). */
rkv_status rkv_append_proj(const rkv_params* p, void* kv, float* ref_proj,
                           const void* kv_new, const int32_t* pos, const void* w1,
                           const void* w2, const void* w3, int32_t* ref_idx,
                           uint8_t* codes, uint16_t* scale, uint16_t* zmin, float* z,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The FP8 reference store of a prefix (p->ref_format == RKV_REF_FP8,
 * [RKV] §2.4 last paragraph): ref_store[b][j][c] = E4M3 byte of
 * kv[b][p_j][c] for the j-th reference position p_j of the schedule, the
 * same values rkv_encode computes with.  kv [B][T][C] in p->dtype (only
 * reference rows are read); ref_store [B][n_ref][C] bytes, n_ref =
 * rkv_reference_positions(p, NULL, 0). */
rkv_status rkv_store_refs(const rkv_params* p, const void* kv, uint8_t* ref_store,
                          hipStream_t stream);

/* The reference schedule of [RKV] §2.6 for p->T, ref_stride, ref_alpha,
 * n_sink, computed on the host (no device work): writes the first
 * min(cap, n) reference positions, ascending, into rpos (HOST memory; may
 * be NULL when cap == 0) and returns n, the number of references per
 * sequence, or -1 on invalid fields (rkv_last_error() says which). */
int32_t rkv_reference_positions(const rkv_params* p, int32_t* rpos,
                                int32_t cap);

/* Observability.  Stages of the encode path, in launch order, plus the
 * gather, the restore and the append.  rkv_profile_begin(mask) makes later
 * calls of this library on this process record a HIP event pair around
 * every stage whose bit (1u << stage) is set in mask, and clears previous
 * records; mask 0 turns recording off (the default).  rkv_profile_read()
 * waits for the recorded events of one stage and returns the summed
 * duration in milliseconds and the number of launches.  Meant for
 * single-threaded measurement; events are created on first use and kept. */
typedef enum {
  RKV_STAGE_PACK = 0,    /* weight repacking on its own (rkv_pack_weights;
                            the restore's decoder weights); none in rkv_encode */
  RKV_STAGE_NORMS = 1,   /* set-up, one launch: weight repacking, schedule
                            tables, reference rows, norms, reference-token
                            records                                         */
  RKV_STAGE_DIST = 2,    /* distance contraction + partial top-k lists; in
                            the encodes the same launch also computes the
                            reference projection P = R [W1|W2]              */
  RKV_STAGE_MERGE = 3,   /* top-k merge, ref_idx of non-reference tokens    */
  RKV_STAGE_PROJ = 4,    /* reserved: the reference projection now runs in
                            the RKV_STAGE_DIST launch; records nothing      */
  RKV_STAGE_SWIGLU = 5,  /* token projection, mean branch, delta_h          */
  RKV_STAGE_W3 = 6,      /* latent z = delta_h W3 + group quantiser         */
  RKV_STAGE_QUANT = 7,   /* stand-alone quantiser (rkv_quantize)            */
  RKV_STAGE_GATHER = 8,  /* gather-dequantise                               */
  RKV_STAGE_RESTORE = 9, /* restore: dequantise, decoder product, mean, RoPE */
  RKV_STAGE_APPEND = 10, /* decode-time append of one token per sequence    */
  RKV_STAGE_STORE = 11,  /* FP8 reference store (rkv_store_refs)            */
  RKV_STAGE_COUNT = 12
} rkv_stage;
rkv_status rkv_profile_begin(uint32_t stage_mask);
rkv_status rkv_profile_read(int32_t stage, double* total_ms, int64_t* launches);

const char* rkv_status_str(rkv_status s);
const char* rkv_last_error(void); /* detail of this thread's last failure */
int rkv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RKV_H */
