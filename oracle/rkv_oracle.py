"""Plain fp64 CPU oracle of the ResidualKV cache-write path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module.  It shares no code with the GPU library
(``reference_residual_encoding_amd``) and neither imports the other; inputs
come from ``synth`` (random draws only).

Source: the ResidualKV reading notes, "ResidualKV：基于参考向量与残差的
KV Cache 压缩" (notes on arXiv 2602.08005v2), cited below as [RKV] with the
notes' own section numbers.  Every step follows the order of [RKV] §2.1-§2.4:

  1. reference schedule: sinks, then p_{m+1} = p_m + s0 +
     floor(alpha (p_m - n_sink)); alpha = 0 is one every s0 tokens ([RKV] §2.6)
  2. candidate pool of token i: earlier references; k_i = min(k, |pool|)
                                                                 ([RKV] §2.1)
  3. the k_i references nearest in squared L2 over the joint vector
                                                  ([RKV] §2.2, retrieval eq.)
  4. their arithmetic mean in KV space           ([RKV] §2.2, mean eq.)
  5. z = f_c(kv_i) - f_c(mean), f_c the SwiGLU compressor
                                          ([RKV] §2.3, f_c and boxed z eq.)
  6. per-token group min-max quantiser            ([RKV] §2.4, three eqs.)
  7. dequantisation of selected tokens           ([RKV] §2.4 third eq.,
                                                   §2.7 decode step 3)

Append (decode step 4 of [RKV] §2.7): a new token at position t is stored as
it is when t is on the schedule, else encoded by steps 2-6 against the
references already in the cache.

Readings taken where the notes are silent (each is listed with its reason in
the design notes of the repository):
  * the schedule starts at p_0 = n_sink after the n_sink sink tokens, which
    are stored as references too; with the defaults (alpha = 0, no sinks)
    references sit at t % s == 0; the pool of token t holds the references at
    positions j < t of the same sequence;
  * distances are unweighted over all 2*d_k coordinates; ties in distance are
    broken by the smaller position;
  * Swish has beta = 1 (SiLU); f_c has no biases;
  * reference tokens are stored as they are: their record is all zero and
    their ref_idx row is all -1;
  * quantiser groups are consecutive coordinates [j*g, (j+1)*g) of one token
    (the last group may be shorter); each group stores two fp16 numbers, the
    step Delta_h = fp16(Delta) and the minimum m_h = fp16(z_min); codes are
    computed against the stored (Delta_h, m_h) so the decoder reproduces the
    encoder's grid, rounded half-to-even and clamped to [0, 2^b - 1]; a group
    whose Delta_h is 0 (constant group) stores q = 0 and decodes to m_h with
    no division;
  * the quantiser decides integers in float32, the precision of the GPU
    kernel: z is rounded to float32 first and (max - min), the division by
    2^b - 1 and (z - m_h) / Delta_h are float32 operations;
  * codes are packed little-endian inside a byte: coordinate r of a byte
    holds bits [r*b, (r+1)*b);
  * dequantised values are q * Delta_h + m_h, exact in float64, then rounded
    once to float32;
  * with quantisation off (b = 16), Q is the identity ([RKV] §2.4): each
    latent is stored as fp16, rounded to nearest even from its float32
    value, and the record holds no group numbers.

Restore (read side, [RKV] §2.5 and the implementation note of §2.1):

  8. for a selected non-reference token: KV^ = z~ W_d + mean of its stored
     references, W_d a bias-free linear map [d_c][2 d_k]; a reference token
     restores to its stored row                          ([RKV] §2.5 boxed eq.)
  9. split KV^ into K (first N*D coordinates) and V; the restored pre-RoPE
     key is rotated at the token's own position                ([RKV] §2.1)

FP8 references ([RKV] §2.4 last paragraph; §2.5: encoder and decoder use
the references as stored): reading, OCP E4M3 (bias 7, 3 mantissa bits,
largest finite 448), round to nearest even, saturating at +-448, no scale
factor; retrieval distances, the mean and the restore all read the FP8
values, the token being encoded its own input row.

Readings for the restore: z~ is the dequantised record of step 7; the
references are the stored rows kv_j at input precision; RoPE pairs
coordinate d of a head with d + D/2 ("rotate half") and turns pair i by
position * theta^(-2i/D), with no frequency scaling; theta <= 0 leaves K
unrotated; an index outside [0, B*T) yields a NaN row.

Parity status: the schedule, selection, mean, compressor, quantiser,
packing, FP8 rounding, restore and append are pinned by the tests in
``tests/test_oracle_pins.py`` (brute force, closed-form identities, special
cases, a library routine and hand-derived golden values; the readings taken
above each have one: the n_sink offset of the schedule, the stored fp16 grid
of the codes, float32 integer decisions, identity-mode rounding).  The
actual numbers of z and of the codes at the synthetic workloads have no
printed counterpart in the pages: beyond those pins they are "parity
unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

F64 = np.float64
F32 = np.float32
IDENTITY_BITS = 16      # b = 16: quantisation off, the latent stored as fp16


# ---------------------------------------------------------------- schedule
def reference_schedule(T: int, s0: int, alpha: float = 0.0, n_sink: int = 0) -> np.ndarray:
    """Reference positions of a sequence of T tokens ([RKV] §2.6).

    The n_sink sink tokens (positions < n_sink) are stored as references;
    then p_0 = n_sink and p_{m+1} = p_m + s0 + floor(alpha * (p_m - n_sink)),
    the floor of the double-precision product.  alpha = 0 is the fixed
    stride s0; with n_sink = 0 as well, the references are t % s0 == 0."""
    pos = list(range(min(n_sink, T)))
    p = n_sink
    while p < T:
        pos.append(p)
        p = p + s0 + math.floor(alpha * (p - n_sink))
    return np.asarray(pos, dtype=np.int64)


def reference_positions(T: int, s: int, alpha: float = 0.0, n_sink: int = 0) -> np.ndarray:
    """The schedule of [RKV] §2.6; fixed stride s by default."""
    return reference_schedule(T, s, alpha, n_sink)


def is_reference(t: int, s: int) -> bool:
    """Fixed-stride schedule (alpha = 0, no sinks): t % s == 0."""
    return t % s == 0


def candidate_pool(t: int, s: int, refs: Optional[np.ndarray] = None) -> np.ndarray:
    """T_ref,t: the references already in the cache when token t is written
    ([RKV] §2.1 symbol table; §2.2 'existing reference pool').  `refs` is the
    sequence's schedule (fixed stride s when None)."""
    if refs is None:
        return np.arange(0, t, s, dtype=np.int64)
    refs = np.asarray(refs, dtype=np.int64)
    return refs[refs < t]


def k_effective(k: int, pool_size: int) -> int:
    """Warm-up neighbour count k_i = min(k, |T_ref,i|) ([RKV] §2.1)."""
    return min(k, pool_size)


# ---------------------------------------------------------------- retrieval
# ---------------------------------------------------------------- FP8 references
FP8_MAX = 448.0


def fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Stored value of a reference coordinate kept in FP8 ([RKV] §2.4 last
    paragraph: references are stored in FP8 in deployment).  Reading: the
    OCP E4M3 format (4 exponent bits, bias 7, 3 mantissa bits, subnormals
    down to 2^-9, largest finite 448, no infinities), round to nearest even,
    saturating at +-448.  Returns float64 values on that grid."""
    x = np.asarray(x, F64)
    a = np.abs(x)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))       # a = m * 2^ex, m in [0.5, 1)
    spacing = np.ldexp(1.0, ex - 1 - 3)               # 3 mantissa bits below the leading one
    r = np.minimum(np.rint(a / spacing) * spacing, FP8_MAX)
    return np.copysign(r, x)


def fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """The E4M3 byte of each value of fp8_e4m3(x): sign, 4-bit biased
    exponent (0 for subnormals), 3-bit mantissa."""
    r = fp8_e4m3(x)
    a = np.abs(r)
    sign = np.where(np.signbit(r), 0x80, 0)
    sub = a < 2.0 ** -6
    _, ex = np.frexp(np.where(sub, 1.0, a))
    e = ex - 1
    mant = np.where(sub, a / 2.0 ** -9, (a / np.ldexp(1.0, e) - 1.0) * 8.0)
    expf = np.where(sub, 0, e + 7)
    return (sign | (expf.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)).astype(np.uint8)


def fp8_e4m3_value(bits: np.ndarray) -> np.ndarray:
    """Value of E4M3 bytes (the inverse of fp8_e4m3_bits on its range)."""
    bits = np.asarray(bits, np.int64)
    sign = np.where(bits & 0x80, -1.0, 1.0)
    e = (bits >> 3) & 0xF
    m = bits & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return sign * val


def stored_references(kv_seq: np.ndarray, refs: np.ndarray, ref_fp8: bool) -> np.ndarray:
    """The cache's view of a sequence: reference rows as stored (FP8 values
    when ref_fp8, else the input rows), every other row as given (never read
    by retrieval or the mean)."""
    out = np.array(kv_seq, dtype=F64, copy=True)
    if ref_fp8 and len(refs):
        out[refs] = fp8_e4m3(out[refs])
    return out


def squared_l2(x: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """||x - y_j||_2^2 for every row y_j of Y, by direct differences."""
    diff = np.asarray(Y, F64) - np.asarray(x, F64)[None, :]
    return np.einsum("jc,jc->j", diff, diff)


def retrieve(kv_seq: np.ndarray, t: int, s: int, k: int, refs: Optional[np.ndarray] = None,
             stored: Optional[np.ndarray] = None):
    """Top-k_t nearest references of token t ([RKV] §2.2 retrieval equation).

    Returns (R, d_sorted): R are the chosen reference positions ordered by
    (distance, position); d_sorted are all pool distances in the same order.
    `stored` holds the references' stored rows (default: kv_seq itself).
    """
    pool = candidate_pool(t, s, refs)
    Y = kv_seq if stored is None else stored
    d = squared_l2(kv_seq[t], Y[pool])
    order = np.lexsort((pool, d))            # primary key d, then position
    k_t = k_effective(k, len(pool))
    return pool[order[:k_t]], d[order]


def reference_mean(kv_seq: np.ndarray, R: Sequence[int]) -> np.ndarray:
    """Arithmetic mean of the retrieved references in KV space ([RKV] §2.2)."""
    return np.asarray(kv_seq[np.asarray(R)], F64).sum(axis=0) / F64(len(R))


# ---------------------------------------------------------------- compressor
def swish(u: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: u * sigmoid(u)."""
    return u / (1.0 + np.exp(-u))


def f_c(x: np.ndarray, W1: np.ndarray, W2: np.ndarray, W3: np.ndarray) -> np.ndarray:
    """SwiGLU compressor (Swish(x W_c1) * x W_c2) W_c3 ([RKV] §2.3), row-wise."""
    x = np.asarray(x, F64)
    return (swish(x @ W1) * (x @ W2)) @ W3


def residual_latent(kv_t, mean, W1, W2, W3) -> np.ndarray:
    """z = f_c(kv_i) - f_c(mean_ref,i) ([RKV] §2.3, boxed equation)."""
    return f_c(kv_t, W1, W2, W3) - f_c(mean, W1, W2, W3)


# ---------------------------------------------------------------- quantiser
def group_bounds(d_c: int, g: int):
    """Consecutive groups of at most g coordinates inside one token ([RKV] §2.4)."""
    return [(a, min(a + g, d_c)) for a in range(0, d_c, g)]


def quantize(z: np.ndarray, g: int, b: int):
    """Per-token group min-max quantiser ([RKV] §2.4).

    z: [n, d_c] latents.  Returns q [n, d_c] (int64 codes), Delta_h and m_h
    [n, n_groups] as float16.  Integer decisions are taken in float32 (see
    the module docstring).  b = 16 is the identity mode: q holds the fp16
    bits of each latent.
    """
    z32 = np.asarray(z, F64).astype(F32)
    n, d_c = z32.shape
    bounds = group_bounds(d_c, g)
    if b == IDENTITY_BITS:
        # quantisation off: Q is the identity map ([RKV] §2.4); the latent is
        # stored as fp16 (round to nearest even from its float32 value) and
        # the record holds no group numbers (zeros here)
        q = z32.astype(np.float16).view(np.uint16).astype(np.int64)
        zeros = np.zeros((n, len(bounds)), dtype=np.float16)
        return q, zeros, zeros.copy()
    levels = F32(2 ** b - 1)
    q = np.zeros((n, d_c), dtype=np.int64)
    dh = np.zeros((n, len(bounds)), dtype=np.float16)
    mh = np.zeros((n, len(bounds)), dtype=np.float16)
    for gi, (a, e) in enumerate(bounds):
        zg = z32[:, a:e]
        zmin = zg.min(axis=1)
        zmax = zg.max(axis=1)
        delta = (zmax - zmin) / levels                 # float32 ops
        dh[:, gi] = delta.astype(np.float16)
        mh[:, gi] = zmin.astype(np.float16)
        dhf = dh[:, gi].astype(F32)[:, None]
        mhf = mh[:, gi].astype(F32)[:, None]
        const = dhf == 0                               # constant group: no division
        safe = np.where(const, F32(1), dhf)
        t = (zg - mhf) / safe
        qq = np.clip(np.rint(t), 0, int(levels)).astype(np.int64)
        q[:, a:e] = np.where(const, 0, qq)
    return q, dh, mh


def dequantize(q: np.ndarray, dh: np.ndarray, mh: np.ndarray, g: int, b: int = 0) -> np.ndarray:
    """z~ = q * Delta + z_min per group ([RKV] §2.4 third equation).

    Exact in float64 for fp16 (Delta_h, m_h) and b <= 8, then one rounding to
    float32.  Returns float32 [n, d_c].  b = 16 (identity mode): the fp16
    value the code holds.
    """
    if b == IDENTITY_BITS:
        return np.asarray(q).astype(np.uint16).view(np.float16).astype(F32)
    n, d_c = q.shape
    out = np.empty((n, d_c), dtype=F64)
    for gi, (a, e) in enumerate(group_bounds(d_c, g)):
        out[:, a:e] = (q[:, a:e].astype(F64) * dh[:, gi:gi + 1].astype(F64)
                       + mh[:, gi:gi + 1].astype(F64))
    return out.astype(F32)


def pack_codes(q: np.ndarray, b: int) -> np.ndarray:
    """Little-endian packing: coordinate per*j + r -> bits [r*b, (r+1)*b) of byte j."""
    n, d_c = q.shape
    if b == IDENTITY_BITS:                               # two bytes per latent, little-endian
        return np.ascontiguousarray(q.astype(np.uint16).astype("<u2")).view(np.uint8).reshape(n, 2 * d_c)
    per = 8 // b
    assert d_c % per == 0
    qq = q.astype(np.uint32).reshape(n, d_c // per, per)
    out = np.zeros((n, d_c // per), dtype=np.uint32)
    for r in range(per):
        out |= qq[:, :, r] << np.uint32(b * r)
    return out.astype(np.uint8)


def unpack_codes(codes: np.ndarray, b: int, d_c: int) -> np.ndarray:
    n = codes.shape[0]
    if b == IDENTITY_BITS:
        return np.ascontiguousarray(codes).view("<u2").reshape(n, d_c).astype(np.int64)
    per = 8 // b
    mask = (1 << b) - 1
    c = codes.astype(np.int64)
    out = np.empty((n, d_c // per, per), dtype=np.int64)
    for r in range(per):
        out[:, :, r] = (c >> (b * r)) & mask
    return out.reshape(n, d_c)


def record_bytes_per_token(d_c: int, g: int, b: int) -> int:
    """b-bit payload plus two fp16 numbers per group ([RKV] §2.4, §3.3)."""
    if b == IDENTITY_BITS:
        return 2 * d_c
    n_groups = -(-d_c // g)
    return d_c * b // 8 + 4 * n_groups


def q_b(b: int, g: int = 32) -> float:
    """Relative group storage vs fp16: b/16 bits-ratio plus two fp16 per g ([RKV] §3.3)."""
    return b / 16.0 + 2.0 / g


def storage_ratio_vs_fp16(C: int, d_c: int, g: int, b: int) -> float:
    """Bytes of one non-reference record over its fp16 joint vector (2*C bytes)."""
    return record_bytes_per_token(d_c, g, b) / (2.0 * C)


def keep_ratio(beta: float, rho_ref: float, qb: float, dc_over_2dk: float,
               q_full: float = None) -> float:
    """KR accounting of [RKV] §3.3: full-attention layers at 4-bit, sparse
    layers holding fp8 references (half of fp16, at density rho_ref) plus the
    short codes."""
    if q_full is None:
        q_full = q_b(4)
    return beta * q_full + (1.0 - beta) * (0.5 * rho_ref + qb * dc_over_2dk)


# ---------------------------------------------------------------- encode
def encode_tokens(kv_seq: np.ndarray, W1, W2, W3, positions: Iterable[int], *,
                  k: int, g: int, b: int, s: int, n_diag: Optional[int] = None,
                  alpha: float = 0.0, n_sink: int = 0, ref_fp8: bool = False) -> Dict:
    """Encode the given positions of one sequence, each on its own.

    kv_seq: [T, C] joint vectors [K heads | V heads], pre-RoPE ([RKV] §2.1).
    Returns per position: ref_idx (sorted positions, -1 pad), z, q, Delta_h,
    m_h, codes, and the first ``n_diag`` pool distances in (d, position)
    order (for the tie rule of the parity tests).
    """
    kv_seq = np.asarray(kv_seq, F64)
    W1 = np.asarray(W1, F64); W2 = np.asarray(W2, F64); W3 = np.asarray(W3, F64)
    positions = np.asarray(list(positions), dtype=np.int64)
    n = len(positions)
    d_c = W3.shape[1]
    if n_diag is None:
        n_diag = k + 1
    ref_idx = np.full((n, k), -1, dtype=np.int32)
    d_diag = np.full((n, n_diag), np.inf)
    z = np.zeros((n, d_c), dtype=F64)
    refs = reference_schedule(len(kv_seq), s, alpha, n_sink)
    ref_mask = np.zeros(len(kv_seq), dtype=bool)
    ref_mask[refs] = True
    # encoder and decoder use the references as stored ([RKV] §2.5), FP8
    # values when they are kept in FP8; the token itself is encoded from its
    # own input row
    stored = stored_references(kv_seq, refs, ref_fp8)
    enc_rows, enc_kv, enc_mean = [], [], []
    for i, t in enumerate(positions):
        if ref_mask[int(t)]:
            continue                       # references are stored as they are
        R, d_sorted = retrieve(kv_seq, int(t), s, k, refs, stored)
        ref_idx[i, :len(R)] = np.sort(R)
        m = min(n_diag, len(d_sorted))
        d_diag[i, :m] = d_sorted[:m]
        enc_rows.append(i)
        enc_kv.append(kv_seq[t])
        enc_mean.append(reference_mean(stored, R))
    if enc_rows:
        rows = np.asarray(enc_rows)
        z[rows] = residual_latent(np.stack(enc_kv), np.stack(enc_mean), W1, W2, W3)
    q, dh, mh = quantize(z, g, b)
    ref_rows = ref_mask[positions]
    q[ref_rows] = 0                        # stored directly: all-zero record
    dh[ref_rows] = 0
    mh[ref_rows] = 0
    return dict(positions=positions, ref_idx=ref_idx, z=z, q=q, scale=dh, zmin=mh,
                codes=pack_codes(q, b), d_diag=d_diag, is_ref=ref_rows)


def encode(kv: np.ndarray, W1, W2, W3, *, k: int, g: int, b: int, s: int,
           alpha: float = 0.0, n_sink: int = 0, ref_fp8: bool = False) -> Dict:
    """Encode every position of every sequence; kv is [B, T, C]."""
    B, T, _ = kv.shape
    parts = [encode_tokens(kv[bi], W1, W2, W3, range(T), k=k, g=g, b=b, s=s, alpha=alpha,
                           n_sink=n_sink, ref_fp8=ref_fp8)
             for bi in range(B)]
    out = {}
    for key in ("ref_idx", "z", "q", "scale", "zmin", "codes", "d_diag", "is_ref"):
        out[key] = np.stack([p[key] for p in parts])
    return out


def append_token(cache_seq: np.ndarray, kv_new: np.ndarray, t: int, W1, W2, W3, *, k: int,
                 g: int, b: int, s: int, alpha: float = 0.0, n_sink: int = 0,
                 ref_fp8: bool = False) -> Dict:
    """Decode step 4 of [RKV] §2.7 for one sequence: the new token enters the
    cache at position t.

    When the schedule ([RKV] §2.6) makes t a reference, the token is stored
    as it is (stored=True, all-zero record, ref_idx all -1).  Otherwise it is
    encoded against the references already in the cache, the rows
    cache_seq[j] at scheduled positions j < t, by retrieval (§2.2), the mean
    (§2.2), z = f_c(kv_new) - f_c(mean) (§2.3) and the quantiser (§2.4).
    No other row of cache_seq is read.  The cache itself is not modified:
    the caller stores stored_row (kv_new, or its FP8 value when ref_fp8) at
    row t when stored is True."""
    T = len(cache_seq)
    kv_new = np.asarray(kv_new, F64)
    d_c = np.asarray(W3).shape[1]
    refs = reference_schedule(T, s, alpha, n_sink)
    ref_idx = np.full(k, -1, dtype=np.int32)
    z = np.zeros((1, d_c), dtype=F64)
    stored = bool(np.any(refs == t))
    if not stored:
        pool = refs[refs < t]
        d = squared_l2(kv_new, np.asarray(cache_seq[pool], F64))
        order = np.lexsort((pool, d))                 # by (distance, position)
        R = pool[order[:k_effective(k, len(pool))]]
        ref_idx[:len(R)] = np.sort(R)
        mean = np.asarray(cache_seq[R], F64).sum(axis=0) / F64(len(R))
        z = residual_latent(kv_new[None, :], mean[None, :], np.asarray(W1, F64),
                            np.asarray(W2, F64), np.asarray(W3, F64))
    q, dh, mh = quantize(z, g, b)
    if stored:
        q[:] = 0
        dh[:] = 0
        mh[:] = 0
    return dict(stored=stored, ref_idx=ref_idx, z=z[0], q=q[0], scale=dh[0], zmin=mh[0],
                codes=pack_codes(q, b)[0],
                stored_row=fp8_e4m3(kv_new) if ref_fp8 else kv_new)


def gather(codes: np.ndarray, scale: np.ndarray, zmin: np.ndarray, idx: np.ndarray,
           *, g: int, b: int, d_c: int) -> np.ndarray:
    """Dequantise only the selected tokens, each from its own record
    ([RKV] §2.4 last paragraph; §2.7 decode step 3).

    codes/scale/zmin are flattened over [B*T]; idx are flat b*T+t indices.
    An index outside [0, B*T) yields a NaN row.
    """
    idx = np.asarray(idx, dtype=np.int64)
    total = codes.shape[0]
    out = np.full((len(idx), d_c), np.nan, dtype=F32)
    ok = (idx >= 0) & (idx < total)
    if ok.any():
        sel = idx[ok]
        q = unpack_codes(codes[sel], b, d_c)
        out[ok] = dequantize(q, scale[sel], zmin[sel], g, b)
    return out


# ---------------------------------------------------------------- restore
def rope_inv_freq(D: int, theta: float) -> np.ndarray:
    """Rotation rate of pair i of a head, theta^(-2i/D), i < D/2 (rotary
    position embedding applied to restored keys, [RKV] §2.1 note)."""
    i = np.arange(D // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * i / F64(D))


def apply_rope(k_flat: np.ndarray, pos: int, N: int, D: int, theta: float) -> np.ndarray:
    """Rotate the N heads of one pre-RoPE key at position `pos`: coordinate d
    and d + D/2 of a head form pair i = d, turned by the angle pos * rate_i."""
    x = np.asarray(k_flat, F64).reshape(N, D)
    if theta <= 0:
        return x.reshape(-1).copy()
    ang = F64(pos) * rope_inv_freq(D, theta)
    c, sn = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, : D // 2], x[:, D // 2:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=1).reshape(-1)


def restore(codes: np.ndarray, scale: np.ndarray, zmin: np.ndarray, ref_idx: np.ndarray,
            kv: np.ndarray, Wd: np.ndarray, idx: np.ndarray, *, s: int, N: int, D: int,
            g: int, b: int, d_c: int, rope_theta: float, alpha: float = 0.0,
            n_sink: int = 0, ref_fp8: bool = False) -> np.ndarray:
    """Restore the selected tokens' K|V rows ([RKV] §2.5): z~ W_d plus the mean
    of the token's stored references, reference tokens as stored; then K is
    rotated at the token's position.

    codes/scale/zmin/ref_idx are flattened over [B*T] (ref_idx rows hold
    reference positions, -1 pads); kv is [B][T][C] (only reference rows are
    read); idx are flat b*T + t.  Returns fp64 [len(idx)][C]; NaN rows for
    indices outside [0, B*T).  With ref_fp8 the references are read as their
    FP8 stored values."""
    Bn, T, C = kv.shape
    refs = reference_schedule(T, s, alpha, n_sink)
    ref_mask = np.zeros(T, dtype=bool)
    ref_mask[refs] = True
    kv = np.stack([stored_references(kv[bq], refs, ref_fp8) for bq in range(Bn)])
    idx = np.asarray(idx, dtype=np.int64)
    out = np.full((len(idx), C), np.nan, dtype=F64)
    Wd = np.asarray(Wd, F64)
    for n, fl in enumerate(idx):
        if fl < 0 or fl >= Bn * T:
            continue
        bq, t = divmod(int(fl), T)
        if ref_mask[t]:
            row = np.asarray(kv[bq, t], F64)
        else:
            q = unpack_codes(codes[fl:fl + 1], b, d_c)
            zt = dequantize(q, scale[fl:fl + 1], zmin[fl:fl + 1], g, b)[0].astype(F64)
            R = [int(p) for p in ref_idx[fl] if p >= 0]
            row = zt @ Wd + reference_mean(kv[bq], R)
        out[n, : N * D] = apply_rope(row[: N * D], t, N, D, rope_theta)
        out[n, N * D:] = row[N * D:]
    return out
