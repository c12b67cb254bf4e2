"""GPU parity of the restore path (rkv_restore, [RKV] §2.5 and the §2.1 note
on rotating restored keys) against the fp64 oracle's restore.

The records (codes, Delta_h, m_h, ref_idx) both sides restore from are the
oracle's own encode of sampled tokens, so nothing the GPU computes feeds the
oracle.  Tolerances (relative L2 per restored row) follow from the
arithmetic: z~ enters the bf16 matrix cores as a (hi, lo) bf16 pair (about
2^-17 relative), W_d is exact, sums are fp32 and sin/cos are fp32 of an fp64
reduced angle, which keeps float output within 2e-5; bf16 output adds one
rounding of at most 2^-9 relative per element, so 4e-3.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import reference_residual_encoding_amd as R
from oracle import rkv_oracle as O
from synth import bf16_bits_to_f32, decoder_weight, generate
from synth.configs import LLAMA8K, LLAMA8K_DYN, LLAMA32K, QWEN_LIKE, TINY, TINY_DYN

import rkv_parity as P

pytestmark = pytest.mark.gpu

REL_F32 = 2e-5
REL_BF16 = 4e-3


def _log(msg):
    print(msg, flush=True)


def _oracle_records(w, positions_by_seq):
    """Records of the sampled tokens by the oracle's encode; zero elsewhere."""
    cfg = w.cfg
    n = cfg.B * cfg.T
    codes = np.zeros((n, cfg.d_c * cfg.b // 8), np.uint8)
    scale = np.zeros((n, cfg.d_c // cfg.g), np.float16)
    zmin = np.zeros_like(scale)
    ref_idx = np.full((n, cfg.k), -1, np.int32)
    kv = w.kv_f32().astype(np.float64)
    W1, W2, W3 = (x.astype(np.float64) for x in w.weights_f32())
    for b, pos in positions_by_seq.items():
        enc = O.encode_tokens(kv[b], W1, W2, W3, pos, k=cfg.k, g=cfg.g, b=cfg.b, s=cfg.stride,
                              alpha=cfg.alpha, n_sink=cfg.n_sink, ref_fp8=cfg.ref_fp8)
        rows = b * cfg.T + np.asarray(enc["positions"])
        codes[rows], scale[rows], zmin[rows], ref_idx[rows] = (
            enc["codes"], enc["scale"], enc["zmin"], enc["ref_idx"])
    return codes, scale, zmin, ref_idx


def _run(w, wd, rec, idx, theta, out_dtype, packed=None):
    cfg = w.cfg
    p = P.params_of(cfg)
    codes, scale, zmin, ref_idx = rec
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d_codes, d_ref = t(codes), t(ref_idx)
    d_scale, d_zmin = t(scale.view(np.int16)), t(zmin.view(np.int16))
    if cfg.ref_fp8:                                  # the E4M3 store [B][nref][C]
        kv = t(P.fp8_store(cfg, w.kv))
    else:
        kv = P.to_device(w.kv, cfg.dtype, dev)
    d_wd = P.to_device(wd, cfg.dtype, dev)
    d_idx = t(np.asarray(idx, np.int32))
    n = len(idx)
    out = torch.empty((max(n, 1), cfg.C), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16,
                      device=dev)
    ws_bytes = R.rkv_restore_workspace_bytes(p, n)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    if packed is None:
        R.rkv_restore(p, d_codes, d_scale, d_zmin, d_ref, kv, d_wd, d_idx, n, theta, out,
                      out_dtype, ws, ws_bytes, stream)
    else:                                   # (buffer, bytes) from rkv_pack_decoder
        R.rkv_restore_packed(p, d_codes, d_scale, d_zmin, d_ref, kv, packed[0], packed[1], d_idx,
                             n, theta, out, out_dtype, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    return out[:n].float().cpu().numpy()


def _oracle(w, wd, rec, idx, theta):
    cfg = w.cfg
    codes, scale, zmin, ref_idx = rec
    return O.restore(codes, scale, zmin, ref_idx, w.kv_f32().astype(np.float64),
                     bf16_bits_to_f32(wd) if cfg.dtype == "bf16" else wd, np.asarray(idx),
                     s=cfg.stride, N=cfg.N, D=cfg.D, g=cfg.g, b=cfg.b, d_c=cfg.d_c,
                     rope_theta=theta, alpha=cfg.alpha, n_sink=cfg.n_sink, ref_fp8=cfg.ref_fp8)


def _compare(got, ref, tol, name):
    ok = ~np.isnan(ref).any(axis=1)
    assert np.array_equal(np.isnan(got).all(axis=1), ~ok), f"{name}: NaN rows differ"
    num = np.linalg.norm(got[ok] - ref[ok], axis=1)
    den = np.linalg.norm(ref[ok], axis=1) + 1e-30
    rel = num / den
    _log(f"[restore] {name}: rows={ok.sum()} rel_max={rel.max() if rel.size else 0:.3e} "
         f"rel_mean={rel.mean() if rel.size else 0:.3e}")
    assert rel.size == 0 or rel.max() <= tol, f"{name}: rel {rel.max():.3e} > {tol}"


@pytest.mark.parametrize("out_dtype,tol", [("f32", REL_F32), ("bf16", REL_BF16)])
def test_restore_tiny_all_positions(out_dtype, tol):
    _log(f"[case] restore tiny_f32 {out_dtype}")
    w = generate(TINY)
    wd = decoder_weight(TINY)
    rec = _oracle_records(w, {0: np.arange(TINY.T)})
    idx = np.arange(TINY.T)
    for theta in (TINY.rope_theta, 0.0):
        got = _run(w, wd, rec, idx, theta, out_dtype)
        _compare(got, _oracle(w, wd, rec, idx, theta), tol, f"tiny theta={theta} {out_dtype}")


@pytest.mark.parametrize("fp8", [False, True])
def test_restore_dynamic_schedule_all_positions(fp8):
    """Sinks and a growing stride ([RKV] §2.6): every reference token,
    sinks included, restores to its own stored row (its FP8 value when the
    references are kept in FP8)."""
    cfg = TINY_DYN.with_(ref_fp8=fp8)
    _log(f"[case] restore {cfg.name}")
    w = generate(cfg)
    wd = decoder_weight(cfg)
    rec = _oracle_records(w, {0: np.arange(cfg.T)})
    idx = np.arange(cfg.T)
    got = _run(w, wd, rec, idx, cfg.rope_theta, "f32")
    _compare(got, _oracle(w, wd, rec, idx, cfg.rope_theta), REL_F32, f"{cfg.name} f32")


@pytest.mark.parametrize("cfg", [LLAMA8K, QWEN_LIKE, LLAMA8K_DYN,
                                 LLAMA8K.with_(name="llama8b_T8k_identity", b=16),
                                 LLAMA8K.with_(name="llama8b_T8k_fp8ref", ref_fp8=True),
                                 LLAMA8K_DYN.with_(name="llama8b_T8k_dynamic_fp8ref", ref_fp8=True)],
                         ids=lambda c: c.name)
def test_restore_sampled_tokens(cfg):
    _log(f"[case] restore {cfg.name}")
    w = generate(cfg)
    wd = decoder_weight(cfg)
    pos = {b: P.sample_positions(cfg.T, cfg.stride, 120, seed=7 + b, cfg=cfg) for b in range(cfg.B)}
    rec = _oracle_records(w, pos)
    idx = np.concatenate([b * cfg.T + pos[b] for b in range(cfg.B)])
    rng = np.random.default_rng(11)
    idx = np.concatenate([idx, rng.choice(idx, 40), [-3, cfg.B * cfg.T]])   # repeats, out of range
    rng.shuffle(idx)
    for out_dtype, tol in (("f32", REL_F32), ("bf16", REL_BF16)):
        got = _run(w, wd, rec, idx, cfg.rope_theta, out_dtype)
        _compare(got, _oracle(w, wd, rec, idx, cfg.rope_theta), tol, f"{cfg.name} {out_dtype}")


@pytest.mark.parametrize("cfg", [LLAMA8K, LLAMA8K_DYN.with_(name="llama8b_T8k_dynamic_fp8ref",
                                                            ref_fp8=True),
                                 LLAMA8K.with_(name="llama8b_T8k_k5", k=5)],
                         ids=lambda c: c.name)
def test_restore_tilings_bit_identical(cfg):
    """The restore runs 256 x 256 tiles (with the rows after their last whole
    round in 128 x 256 tiles of the same launch), or 128 x 128 tiles two to
    a CU where the wide ones would fill at most half the CUs;
    RKV_RESTORE_TILE forces every row into wide tiles, into the small 8-wave
    tiles, into the 4-wave ones, or a split after 256 rows.  The tile shape
    changes no output's arithmetic, so all give the same bits, in f32 and
    bf16, with FP8 references and k > 4."""
    import os
    w = generate(cfg)
    wd = decoder_weight(cfg)
    pos = {b: P.sample_positions(cfg.T, cfg.stride, 200, seed=3 + b, cfg=cfg) for b in range(cfg.B)}
    rec = _oracle_records(w, pos)
    idx = np.concatenate([b * cfg.T + pos[b] for b in range(cfg.B)] + [[-1, 5]])
    assert len(idx) > 256
    for out_dtype in ("f32", "bf16"):
        got = {}
        for tiling in ("wide", "tail", "narrow", "256"):
            os.environ["RKV_RESTORE_TILE"] = tiling
            try:
                got[tiling] = _run(w, wd, rec, idx, cfg.rope_theta, out_dtype)
            finally:
                del os.environ["RKV_RESTORE_TILE"]
        for tiling in ("tail", "narrow", "256"):
            assert np.array_equal(got["wide"].view(np.uint32), got[tiling].view(np.uint32)), \
                (out_dtype, tiling)


@pytest.mark.parametrize("cfg", [LLAMA8K, LLAMA8K_DYN.with_(name="llama8b_T8k_dynamic_fp8ref",
                                                            ref_fp8=True)],
                         ids=lambda c: c.name)
def test_restore_packed_matches_restore(cfg):
    """rkv_restore_packed with the buffer rkv_pack_decoder writes gives
    exactly rkv_restore's rows (f32 and bf16 output), across two calls that
    reuse the packed buffer."""
    w = generate(cfg)
    wd = decoder_weight(cfg)
    pos = {b: P.sample_positions(cfg.T, cfg.stride, 150, seed=21 + b, cfg=cfg) for b in range(cfg.B)}
    rec = _oracle_records(w, pos)
    idx = np.concatenate([b * cfg.T + pos[b] for b in range(cfg.B)] + [[-1, 7]])
    p = P.params_of(cfg)
    d_wd = P.to_device(wd, cfg.dtype, "cuda")
    nbytes = R.rkv_packed_decoder_bytes(p)
    packed = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    R.rkv_pack_decoder(p, d_wd, packed, nbytes, torch.cuda.current_stream().cuda_stream)
    for out_dtype in ("f32", "bf16"):
        want = _run(w, wd, rec, idx, cfg.rope_theta, out_dtype)
        got = _run(w, wd, rec, idx, cfg.rope_theta, out_dtype, packed=(packed, nbytes))
        assert np.array_equal(want.view(np.uint32), got.view(np.uint32)), out_dtype


def test_restore_reference_rows_exact_without_rotation():
    """References are stored as they are ([RKV] §2.4): unrotated, their
    restore is the stored row, bit for bit."""
    cfg = LLAMA8K
    w = generate(cfg)
    wd = decoder_weight(cfg)
    refs = np.arange(0, 2048, cfg.stride)
    rec = _oracle_records(w, {0: np.array([1, 17])})
    got = _run(w, wd, rec, refs, 0.0, "f32")
    np.testing.assert_array_equal(got, w.kv_f32()[0, refs])


def test_restore_bench_shape_sampled():
    """The gather subset of the long-context workload, in the benchmark's
    launch shape (9,830 rows), checked on a sample the oracle can encode."""
    cfg = LLAMA32K
    _log("[case] restore llama8b_T32k bench shape")
    w = generate(cfg)
    wd = decoder_weight(cfg)
    idx = w.gather_idx.astype(np.int64)
    sample = np.sort(np.random.default_rng(5).choice(idx, 160, replace=False))
    rec = _oracle_records(w, {0: sample})
    got = _run(w, wd, rec, idx, cfg.rope_theta, "bf16")
    where = np.searchsorted(idx, sample)
    _compare(got[where], _oracle(w, wd, rec, sample, cfg.rope_theta), REL_BF16, "llama8b_T32k bf16")


def test_restore_empty_is_a_no_op():
    cfg = TINY
    p = P.params_of(cfg)
    assert R.rkv_restore(p, None, None, None, None, None, None, None, 0, 1.0, None, "f32",
                         None, 0, None) == 0
