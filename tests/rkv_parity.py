"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the fp64 CPU oracle on the same seeded inputs.

Tolerances (per token unless stated):
  * reference sets identical, except where the oracle's k-th and (k+1)-th
    distances differ but lie within 1e-4 relative of each other (several
    answers are then correct; an exact tie is not excused): there the GPU's set must still be a valid top-k (every
    chosen reference no farther than the oracle's k-th distance, within the
    same 1e-4), and z / codes are compared with the oracle re-run on the
    GPU's set;
  * latent z within 1e-2 relative L2;
  * codes identical on >= 99.9 % of entries, the others off by exactly 1;
    in identity mode (quantisation off) the codes are the fp16 bits of z:
    each side rounds its own z, which agree to ~1e-6 of the token's norm,
    so a coordinate small against the norm may sit several fp16 ulps apart;
    there every stored latent is held to one fp16 ulp plus the z bar, and
    the dequantised bars below count every coordinate;
  * dequantised latents within 1e-2 relative L2: per token on the
    coordinates whose codes agree, and over the whole sample; a coordinate
    whose code is off by one differs by at most one quantisation step.
"""
from __future__ import annotations

import numpy as np
import torch

import reference_residual_encoding_amd as R
from reference_residual_encoding_amd import buffers as RB
from oracle import rkv_oracle as O
from synth import f32_to_bf16_bits

TIE_REL = 1e-4
Z_REL = 1e-2
CODE_MATCH = 0.999
DEQ_REL = 1e-2


def params_of(cfg):
    return R.params(B=cfg.B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k,
                    g=cfg.g, b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
                    ref_alpha=cfg.alpha, ref_format="fp8" if cfg.ref_fp8 else "input")


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def run_encode(w, device="cuda", with_z=True):
    cfg = w.cfg
    p = params_of(cfg)
    kv = to_device(w.kv, cfg.dtype, device)
    w1, w2, w3 = (to_device(x, cfg.dtype, device) for x in (w.w1, w.w2, w.w3))
    out = RB.alloc_encode(p, device, with_z)
    RB.encode(p, kv, w1, w2, w3, out)
    torch.cuda.synchronize()
    host = dict(ref_idx=out.ref_idx.cpu().numpy(), codes=out.codes.cpu().numpy(),
                scale=out.scale.cpu().numpy(), zmin=out.zmin.cpu().numpy(),
                z=out.z.cpu().numpy() if with_z else None)
    return p, out, host, (kv, w1, w2, w3)


def fp8_store(cfg, kv_bits: np.ndarray) -> np.ndarray:
    """The FP8 reference store [B][nref][C] of a prefix, built on the host
    from the format (the oracle's E4M3 rounding)."""
    refs = O.reference_schedule(cfg.T, cfg.stride, cfg.alpha, cfg.n_sink)
    kv = kv_bits_to_f64(cfg, kv_bits)
    return O.fp8_e4m3_bits(kv[:, refs])


def kv_bits_to_f64(cfg, kv_bits: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return (kv_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return kv_bits.astype(np.float64)


def ref_mask_of(cfg) -> np.ndarray:
    """Boolean [T]: the positions the schedule stores as references."""
    m = np.zeros(cfg.T, dtype=bool)
    m[O.reference_schedule(cfg.T, cfg.stride, cfg.alpha, cfg.n_sink)] = True
    return m


def sample_positions(T: int, s: int, n_random: int, seed: int = 123, cfg=None) -> np.ndarray:
    """Warm-up, tail, token-tile boundaries (tiles of 128 non-reference
    tokens) and n_random seeded positions."""
    rng = np.random.default_rng(seed)
    mask = ref_mask_of(cfg) if cfg is not None else (np.arange(T) % s) == 0
    refs, nonref = np.flatnonzero(mask), np.flatnonzero(~mask)
    n_sink = cfg.n_sink if cfg is not None else 0
    warm = int(refs[min(len(refs) - 1, n_sink + 3)]) + 8
    pos = set(range(min(T, warm)))                      # warm-up: k_t < k, references
    pos |= set(range(max(0, T - 24), T))                # tail
    for q in range(0, len(nonref), 128):
        for dq in (-1, 0, 1):
            if 0 <= q + dq < len(nonref):
                pos.add(int(nonref[q + dq]))
    pos |= set(int(x) for x in rng.choice(T, size=min(T, n_random), replace=False))
    return np.array(sorted(p for p in pos if p < T), dtype=np.int64)


def compare_tokens(w, host, positions_by_seq, gathered=None, log=print):
    """Check the GPU record of the given positions against the oracle.

    positions_by_seq: {b: positions}.  gathered: optional {b: GPU
    dequantised rows for those positions} (float32).  Returns a summary."""
    cfg = w.cfg
    k, g, bb, s = cfg.k, cfg.g, cfg.b, cfg.stride
    kv32 = w.kv_f32()
    W1, W2, W3 = (x.astype(np.float64) for x in w.weights_f32())
    n_tok = n_excused = n_diff_set = 0
    code_total = code_equal = 0
    max_code_diff = 0
    z_rel_max = deq_rel_max = 0.0
    deq_num2 = deq_den2 = 0.0
    for bi, pos in positions_by_seq.items():
        kvb = kv32[bi].astype(np.float64)
        orc = O.encode_tokens(kvb, W1, W2, W3, pos, k=k, g=g, b=bb, s=s, alpha=cfg.alpha,
                              n_sink=cfg.n_sink, ref_fp8=cfg.ref_fp8)
        stored = O.stored_references(kvb, O.reference_schedule(cfg.T, s, cfg.alpha, cfg.n_sink),
                                     cfg.ref_fp8)
        g_ref = host["ref_idx"][bi, pos]
        z_orc = orc["z"].copy()
        for i, t in enumerate(pos):
            if orc["is_ref"][i]:
                assert np.all(g_ref[i] == -1), (bi, t)
                assert np.all(host["codes"][bi, t] == 0)
                if bb != O.IDENTITY_BITS:
                    assert np.all(host["scale"][bi, t] == 0) and np.all(host["zmin"][bi, t] == 0)
                if host["z"] is not None:
                    assert np.all(host["z"][bi, t] == 0)
                continue
            n_tok += 1
            o_set = orc["ref_idx"][i]
            k_t = int((o_set >= 0).sum())
            gs = g_ref[i]
            assert int((gs >= 0).sum()) == k_t, (bi, t, gs, o_set)
            assert np.all(gs[k_t:] == -1) and np.all(np.diff(gs[:k_t]) > 0), (bi, t, gs)
            if not np.array_equal(np.sort(gs[:k_t]), np.sort(o_set[:k_t])):
                n_diff_set += 1
                dk, dk1 = orc["d_diag"][i, k_t - 1], orc["d_diag"][i, k_t]
                # near-ties only: an exact tie (dk1 == dk, e.g. two equal
                # reference rows) has one right answer, the smaller position
                excused = np.isfinite(dk1) and dk1 != dk and abs(dk1 - dk) <= TIE_REL * abs(dk)
                assert excused, f"seq {bi} token {t}: GPU set {gs} vs oracle {o_set} (d_k={dk}, d_k+1={dk1})"
                d_gpu = O.squared_l2(kvb[t], stored[gs[:k_t]])
                assert np.all(d_gpu <= dk * (1 + TIE_REL)), (bi, t, d_gpu, dk)
                z_orc[i] = O.residual_latent(kvb[t], O.reference_mean(stored, gs[:k_t]), W1, W2, W3)
                n_excused += 1
        q_orc, dh_orc, mh_orc = O.quantize(z_orc, g, bb)
        q_orc[orc["is_ref"]] = 0
        dh_orc[orc["is_ref"]] = 0
        mh_orc[orc["is_ref"]] = 0
        nonref = ~orc["is_ref"]
        if host["z"] is not None:
            zg = host["z"][bi, pos].astype(np.float64)
            num = np.linalg.norm(zg - z_orc, axis=1)[nonref]
            den = np.maximum(np.linalg.norm(z_orc, axis=1)[nonref], 1e-30)
            if num.size:
                z_rel_max = max(z_rel_max, float((num / den).max()))
        q_gpu = O.unpack_codes(host["codes"][bi, pos], bb, cfg.d_c)
        diff = np.abs(q_gpu - q_orc)[nonref]
        code_total += diff.size
        code_equal += int((diff == 0).sum())
        if diff.size:
            max_code_diff = max(max_code_diff, int(diff.max()))
        deq_orc = O.dequantize(q_orc, dh_orc, mh_orc, g, bb).astype(np.float64)
        if gathered is not None:
            deq_gpu = gathered[bi].astype(np.float64)
        else:
            deq_gpu = O.dequantize(q_gpu, host["scale"][bi, pos], host["zmin"][bi, pos], g, bb)
        # A code off by one (allowed above) moves its coordinate by one step
        # Delta_h, itself ~2 % (INT4) to ~6 % (INT2) of a token's norm; so
        # the dequantised bound is per token on the coordinates whose codes
        # agree, over the whole sample (relative Frobenius), and one step
        # (plus the fp16 record's own difference) on the flipped ones.
        agree = (q_gpu == q_orc)
        err = deq_gpu - deq_orc
        # identity mode: every stored latent counts (no code flips to set aside)
        counted = np.ones_like(agree) if bb == O.IDENTITY_BITS else agree
        num = np.linalg.norm(np.where(counted, err, 0.0), axis=1)[nonref]
        den = np.maximum(np.linalg.norm(deq_orc, axis=1)[nonref], 1e-30)
        if num.size:
            deq_rel_max = max(deq_rel_max, float((num / den).max()))
        deq_num2 += float((err[nonref] ** 2).sum())
        deq_den2 += float((deq_orc[nonref] ** 2).sum())
        flip = ~agree & nonref[:, None]
        if flip.any() and bb == O.IDENTITY_BITS:
            # identity mode: each side rounds its own z to fp16, so a stored
            # latent may differ by one fp16 ulp (2^-10 relative) plus the two
            # z's own difference, which the z bar bounds by Z_REL of the
            # token's norm (a coordinate far below the norm can then sit
            # several ulps apart)
            zn = np.linalg.norm(z_orc, axis=1)[:, None]
            lim = np.maximum(np.abs(deq_orc), np.abs(deq_gpu)) * 2.0 ** -10 + 2.0 ** -24 + Z_REL * zn
            assert np.all(np.abs(err)[flip] <= lim[flip]), "fp16 latent outside one ulp + the z bar"
        elif flip.any():
            step_o = np.repeat(dh_orc.astype(np.float64), g, axis=1)
            step_g = np.repeat(host["scale"][bi, pos].astype(np.float64), g, axis=1)
            mdiff = np.abs(np.repeat(host["zmin"][bi, pos].astype(np.float64) - mh_orc.astype(np.float64), g, axis=1))
            lim = np.maximum(step_o, step_g) * 1.001 + mdiff + 16 * np.abs(step_g - step_o)
            assert np.all(np.abs(err)[flip] <= lim[flip]), "flipped code moved more than one step"
        if gathered is not None:
            assert np.all(gathered[bi][orc["is_ref"]] == 0)
    match = code_equal / code_total if code_total else 1.0
    deq_rel_all = float(np.sqrt(deq_num2 / max(deq_den2, 1e-300)))
    summary = dict(tokens=n_tok, set_diff=n_diff_set, excused=n_excused, z_rel_max=z_rel_max,
                   code_match=match, max_code_diff=max_code_diff, deq_rel_max=deq_rel_max,
                   deq_rel_all=deq_rel_all)
    log(f"[parity] {cfg.name}: {summary}")
    assert z_rel_max <= Z_REL, summary
    if bb != O.IDENTITY_BITS:
        assert match >= CODE_MATCH, summary
        assert max_code_diff <= 1, summary
    assert deq_rel_max <= DEQ_REL, summary
    assert deq_rel_all <= DEQ_REL, summary
    return summary


def check_record_invariants(cfg, host):
    """Properties that hold at any size, checked on every token."""
    B, T, k = cfg.B, cfg.T, cfg.k
    t = np.arange(T)
    is_ref = ref_mask_of(cfg)
    pool = np.cumsum(is_ref) - is_ref                       # references before t
    want = np.where(is_ref, 0, np.minimum(k, pool))
    ri = host["ref_idx"]
    cnt = (ri >= 0).sum(axis=2)
    assert np.array_equal(cnt, np.broadcast_to(want, (B, T)))
    valid = ri >= 0
    assert np.all(is_ref[ri[valid]])                        # members of the schedule
    assert np.all(np.where(valid, ri, -1) < t[None, :, None])
    assert np.all(valid[:, :, 1:] <= valid[:, :, :-1])          # chosen first, then pads
    both = valid[:, :, 1:] & valid[:, :, :-1]
    assert np.all(np.diff(ri, axis=2)[both] > 0)                # ascending positions
    assert np.all(host["codes"][:, is_ref] == 0)
    if cfg.b != O.IDENTITY_BITS:
        assert np.all(host["scale"][:, is_ref] == 0) and np.all(host["zmin"][:, is_ref] == 0)


def check_quantizer_bit_exact(cfg, host):
    """The encode's codes/scale/zmin are the quantiser applied to its own z:
    compare with the oracle quantiser on that same float32 z, bit for bit."""
    z = host["z"].reshape(-1, cfg.d_c)
    q, dh, mh = O.quantize(z.astype(np.float64), cfg.g, cfg.b)
    codes = host["codes"].reshape(len(z), -1)
    assert np.array_equal(codes, O.pack_codes(q, cfg.b))
    if cfg.b == O.IDENTITY_BITS:
        return
    assert np.array_equal(host["scale"].reshape(len(z), -1).view(np.uint16), dh.view(np.uint16))
    assert np.array_equal(host["zmin"].reshape(len(z), -1).view(np.uint16), mh.view(np.uint16))


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def expected_bf16(x32: np.ndarray) -> np.ndarray:
    out = f32_to_bf16_bits(np.nan_to_num(x32, nan=0.0))
    return out
