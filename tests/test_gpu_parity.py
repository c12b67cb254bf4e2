"""GPU parity: the HIP path (called through the C ABI) against the fp64 CPU
oracle on the same seeded inputs.  Needs an MI355X."""
import os
import numpy as np
import pytest
import torch

import reference_residual_encoding_amd as R
from reference_residual_encoding_amd import buffers as RB
from oracle import rkv_oracle as O
from synth import generate
from synth.configs import (LLAMA8K, LLAMA8K_DYN, LLAMA32K, LLAMA32K_DYN, MM_INT2, QWEN_LIKE,
                           TINY, TINY_DYN)

import rkv_parity as P

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _gather_rows(p, out, idx_flat):
    idx = torch.from_numpy(np.asarray(idx_flat, dtype=np.int32)).cuda()
    rows = RB.dequant_gather(p, out, idx, "f32")
    torch.cuda.synchronize()
    return rows.cpu().numpy()


def _full_parity(cfg):
    w = generate(cfg)
    p, out, host, _ = P.run_encode(w)
    P.check_record_invariants(cfg, host)
    P.check_quantizer_bit_exact(cfg, host)
    pos = {b: np.arange(cfg.T) for b in range(cfg.B)}
    gathered = {b: _gather_rows(p, out, b * cfg.T + pos[b]) for b in range(cfg.B)}
    return P.compare_tokens(w, host, pos, gathered, log=_log)


def test_tiny_f32_all_positions():
    _log("[case] tiny_f32 full")
    _full_parity(TINY)


# Ragged shapes spanning several tiles, non-power-of-two stride, k > 4
# (8-long neighbour lists), g = 16 and 64, INT2, both dtypes.
RAGGED = [
    LLAMA8K.with_(name="ragged_bf16_b2_k5", B=3, T=1000, N=2, D=32, d_ff=96, d_c=64, k=5, g=16,
                  b=2, stride=7, n_protos=24),
    LLAMA8K.with_(name="ragged_f32_k1_g64", B=2, T=777, N=1, D=64, d_ff=64, d_c=128, k=1, g=64,
                  b=4, stride=3, dtype="f32", n_protos=12, noise=0.3),
    LLAMA8K.with_(name="ragged_bf16_k8_g8", B=1, T=1300, N=4, D=32, d_ff=160, d_c=96, k=8, g=8,
                  b=4, stride=16, n_protos=40),
]


@pytest.mark.parametrize("cfg", RAGGED, ids=lambda c: c.name)
def test_ragged_shapes_all_positions(cfg):
    _log(f"[case] {cfg.name} full")
    _full_parity(cfg)


EDGE = [
    TINY.with_(name="edge_T1", T=1),
    TINY.with_(name="edge_T_lt_s", T=5),
    TINY.with_(name="edge_T_eq_s_plus1", T=9),
    TINY.with_(name="edge_s1_all_refs", T=40, stride=1),
    TINY.with_(name="edge_s_gt_T", T=20, stride=64),
    TINY.with_(name="edge_bf16_T130", T=130, dtype="bf16"),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_edge_cases(cfg):
    _log(f"[case] {cfg.name}")
    _full_parity(cfg)


@pytest.mark.parametrize("cfg,n_random", [(LLAMA8K, 800), (LLAMA32K, 500), (QWEN_LIKE, 300),
                                          (MM_INT2, 200)], ids=lambda c: getattr(c, "name", c))
def test_full_size_configs_sampled(cfg, n_random):
    """Full-size workloads, in the launch configuration the benchmark times:
    invariants and bit-exact quantiser on every token, oracle parity on a
    sample of tokens computed one by one."""
    _log(f"[case] {cfg.name} sampled")
    w = generate(cfg)
    p, out, host, _ = P.run_encode(w)
    P.check_record_invariants(cfg, host)
    P.check_quantizer_bit_exact(cfg, host)
    pos = {b: P.sample_positions(cfg.T, cfg.stride, n_random, seed=100 + b, cfg=cfg)
           for b in range(cfg.B)}
    gathered = {b: _gather_rows(p, out, b * cfg.T + pos[b]) for b in range(cfg.B)}
    P.compare_tokens(w, host, pos, gathered, log=_log)
    if cfg.gather_frac is not None:
        _check_configured_gather(w, p, out, host)


def _check_configured_gather(w, p, out, host):
    """The workload's own gather (a random 30 % or 10 % of the flat token
    indices, sorted): every row bit-exact in f32 and bf16 against the
    oracle's dequantisation of the GPU's records ([RKV] §2.4 third eq.)."""
    cfg = w.cfg
    idx = np.asarray(w.gather_idx, dtype=np.int32)
    d_idx = torch.from_numpy(idx).cuda()
    got32 = RB.dequant_gather(p, out, d_idx, "f32")
    got16 = RB.dequant_gather(p, out, d_idx, "bf16")
    torch.cuda.synchronize()
    flat = lambda a: a.reshape(cfg.B * cfg.T, -1)
    want = O.gather(flat(host["codes"]), flat(host["scale"]), flat(host["zmin"]), idx,
                    g=cfg.g, b=cfg.b, d_c=cfg.d_c)
    _log(f"[gather] {cfg.name}: {len(idx)} rows")
    assert np.array_equal(got32.cpu().numpy(), want)
    assert np.array_equal(P.bf16_bits_of(got16), P.expected_bf16(want))


# Dynamic reference schedule ([RKV] §2.6): sinks, a growing stride, a pool
# that outgrows one candidate chunk, schedules where the sinks cover the
# whole sequence, both dtypes.
DYN_EDGE = [
    TINY_DYN,
    TINY.with_(name="dyn_sinks_cover_T", T=6, n_sink=8, alpha=0.1),
    TINY.with_(name="dyn_sinks_fixed_stride", T=200, n_sink=5),
    TINY.with_(name="dyn_fast_growth_bf16", T=500, alpha=0.5, n_sink=1, dtype="bf16"),
    RAGGED[0].with_(name="dyn_ragged_bf16_k5", alpha=0.01, n_sink=3),
    RAGGED[2].with_(name="dyn_ragged_bf16_k8", T=3000, stride=2, alpha=0.002, n_sink=16),
]


@pytest.mark.parametrize("cfg", DYN_EDGE, ids=lambda c: c.name)
def test_dynamic_schedule_all_positions(cfg):
    _log(f"[case] {cfg.name} full")
    _full_parity(cfg)


@pytest.mark.parametrize("cfg,n_random", [(LLAMA8K_DYN, 600), (LLAMA32K_DYN, 400)],
                         ids=lambda c: getattr(c, "name", c))
def test_dynamic_schedule_sampled(cfg, n_random):
    test_full_size_configs_sampled(cfg, n_random)


# Quantisation off ([RKV] §2.4: Q is the identity; the latent stored as fp16).
IDENTITY = [
    TINY.with_(name="tiny_f32_identity", b=16),
    RAGGED[0].with_(name="ragged_bf16_identity_dynamic", b=16, alpha=0.01, n_sink=3),
]


@pytest.mark.parametrize("cfg", IDENTITY, ids=lambda c: c.name)
def test_identity_mode_all_positions(cfg):
    _log(f"[case] {cfg.name} full")
    _full_parity(cfg)


def test_identity_mode_sampled():
    test_full_size_configs_sampled(LLAMA8K.with_(name="llama8b_T8k_identity", b=16), 400)


# FP8 references ([RKV] §2.4 last paragraph; §2.5: the encoder uses them as
# stored): retrieval and the mean read their E4M3 values.
FP8 = [
    TINY.with_(name="tiny_f32_fp8ref", ref_fp8=True),
    RAGGED[0].with_(name="ragged_bf16_fp8ref_dynamic", ref_fp8=True, alpha=0.01, n_sink=3),
    RAGGED[2].with_(name="ragged_bf16_fp8ref_k8_identity", ref_fp8=True, b=16),
]


@pytest.mark.parametrize("cfg", FP8, ids=lambda c: c.name)
def test_fp8_references_all_positions(cfg):
    _log(f"[case] {cfg.name} full")
    _full_parity(cfg)


def test_fp8_references_sampled():
    test_full_size_configs_sampled(LLAMA8K.with_(name="llama8b_T8k_fp8ref", ref_fp8=True), 400)


@pytest.mark.parametrize("cfg", [
    TINY.with_(name="store_f32", ref_fp8=True),
    LLAMA8K.with_(name="store_bf16_B2", B=2, T=2048, ref_fp8=True),
    # a growing schedule (still stride 2 below 5,005) with 2,003 references:
    # three chunks of host positions in the kernel arguments
    LLAMA8K.with_(name="store_bf16_dynamic", T=4000, stride=2, alpha=0.0002, n_sink=5,
                  ref_fp8=True),
], ids=lambda c: c.name)
def test_fp8_store_is_bit_exact(cfg):
    """rkv_store_refs writes the E4M3 bytes of every reference row, as the
    format rounds them (the oracle's rounding), in schedule order."""
    _log(f"[case] store {cfg.name}")
    w = generate(cfg)
    p = P.params_of(cfg)
    refs = R.rkv_reference_positions(p)
    kv = P.to_device(w.kv, cfg.dtype)
    store = torch.full((cfg.B, len(refs), cfg.C), 0xAB, dtype=torch.uint8, device="cuda")
    R.rkv_store_refs(p, kv, store, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(store.cpu().numpy(), P.fp8_store(cfg, w.kv))


@pytest.mark.parametrize("cfg", [TINY, RAGGED[0], RAGGED[1], LLAMA8K.with_(T=4096),
                                 LLAMA8K_DYN.with_(name="llama_dyn_fp8_identity", T=3000,
                                                   ref_fp8=True, b=16)],
                         ids=lambda c: c.name)
def test_encode_packed_matches_encode(cfg):
    """rkv_encode_packed with weights packed once by rkv_pack_weights gives
    rkv_encode's outputs bit for bit, on two calls with one packed buffer."""
    _log(f"[case] packed {cfg.name}")
    w = generate(cfg)
    p, _, h1, (kv, w1, w2, w3) = P.run_encode(w)
    packed = RB.pack_weights(p, w1, w2, w3)
    for rep in range(2):
        out = RB.alloc_encode(p, "cuda", True)
        RB.encode_packed(p, kv, packed, out)
        torch.cuda.synchronize()
        h2 = dict(ref_idx=out.ref_idx.cpu().numpy(), codes=out.codes.cpu().numpy(),
                  scale=out.scale.cpu().numpy(), zmin=out.zmin.cpu().numpy(),
                  z=out.z.cpu().numpy())
        for key in ("ref_idx", "codes", "scale", "zmin", "z"):
            assert np.array_equal(h1[key].view(np.uint8), h2[key].view(np.uint8)), (rep, key)


def test_select_export_matches_encode():
    cfg = LLAMA8K.with_(T=2048)
    w = generate(cfg)
    p, out, host, (kv, *_) = P.run_encode(w, with_z=False)
    ri = torch.empty_like(out.ref_idx)
    R.rkv_select(p, kv, ri, out.workspace, out.workspace.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(ri.cpu().numpy(), host["ref_idx"])


def test_encode_is_deterministic():
    cfg = LLAMA8K.with_(T=4096)
    w = generate(cfg)
    _, _, h1, _ = P.run_encode(w)
    _, _, h2, _ = P.run_encode(w)
    for key in ("ref_idx", "codes", "scale", "zmin", "z"):
        assert np.array_equal(h1[key].view(np.uint8), h2[key].view(np.uint8)), key


@pytest.mark.parametrize("cfg", [LLAMA8K.with_(name="llama_B3_T1500", B=3, T=1500),
                                 LLAMA8K_DYN.with_(name="llama_dyn_B2_T3000", B=2, T=3000)],
                         ids=lambda c: c.name)
def test_encode_dma_forms_bit_identical(cfg):
    """The contractions over kv rows copy operands to LDS through buffer
    resources (32-bit offsets from each tile's first row) unless a tile spans
    2 GB; RKV_DMA_GLOBAL=1 forces the 64-bit-address form.  Both must give
    the same bits, including token tiles that cross from one sequence into
    the next (B > 1, nr not a multiple of the tile)."""
    w = generate(cfg)
    _, _, h1, _ = P.run_encode(w)
    os.environ["RKV_DMA_GLOBAL"] = "1"
    try:
        _, _, h2, _ = P.run_encode(w)
    finally:
        del os.environ["RKV_DMA_GLOBAL"]
    for key in ("ref_idx", "codes", "scale", "zmin", "z"):
        assert np.array_equal(h1[key].view(np.uint8), h2[key].view(np.uint8)), key



@pytest.mark.parametrize("cfg", [LLAMA8K.with_(name="llama_B3_T1500", B=3, T=1500), RAGGED[0],
                                 RAGGED[1]], ids=lambda c: c.name)
def test_swiglu_tile_orders_bit_identical(cfg):
    """k_swiglu runs its tiles row tile fastest, or column tile fastest once
    the kv rows outgrow the MALL; RKV_SWIGLU_ORDER forces either.  The order
    only moves work between workgroups, so both give the same bits, with
    ragged column tiles (d_ff = 96, 64) and token tiles that cross sequences.
    delta_h is written non-temporally once it outgrows the caches;
    RKV_DH_NT forces either, with the same bits."""
    outs = []
    for order, nt in (("row", "0"), ("col", "0"), ("row", "1")):
        os.environ["RKV_SWIGLU_ORDER"] = order
        os.environ["RKV_DH_NT"] = nt
        try:
            _, _, h, _ = P.run_encode(generate(cfg))
        finally:
            del os.environ["RKV_SWIGLU_ORDER"]
            del os.environ["RKV_DH_NT"]
        outs.append(h)
    for key in ("ref_idx", "codes", "scale", "zmin", "z"):
        for other in outs[1:]:
            assert np.array_equal(outs[0][key].view(np.uint8), other[key].view(np.uint8)), key


@pytest.mark.parametrize("cfg", [LLAMA8K.with_(name="llama_B3_T1500", B=3, T=1500), RAGGED[0],
                                 RAGGED[2], LLAMA8K_DYN.with_(name="llama_dyn_B2_T3000", B=2,
                                                              T=3000)],
                         ids=lambda c: c.name)
def test_distance_tilings_bit_identical(cfg):
    """The distance launch runs wide tiles (8 waves, 256 tokens), narrow
    ones (4 waves, 128 tokens, two workgroups per CU), or narrow ones on
    128-reference chunks, as the shape asks; RKV_DIST_TILE forces any.  The
    tilings only group each token's candidates into lists differently, and
    the merge orders them by (d, j), so all outputs (and the reference
    projection that rides in the same launch) are the same bits, for k = 4
    and k > 4 lists, a growing schedule and several sequences.  Rows of a
    chunk that no token of its tile may use read a zero row; with
    RKV_DIST_ZERO=0 they repeat a reference row instead, and the bits stay
    the same (those products are masked).  Token tiles go to the XCDs in
    turn or in serpentine order (RKV_DIST_DEAL), with the same bits."""
    outs = []
    for tiling, extra in (("wide", {}), ("narrow", {}), ("short", {}),
                          ("wide", {"RKV_DIST_ZERO": "0"}), ("short", {"RKV_DIST_ZERO": "0"}),
                          ("wide", {"RKV_DIST_DEAL": "serp"}),
                          ("narrow", {"RKV_DIST_DEAL": "turn"})):
        os.environ["RKV_DIST_TILE"] = tiling
        os.environ.update(extra)
        try:
            _, _, h, _ = P.run_encode(generate(cfg))
        finally:
            del os.environ["RKV_DIST_TILE"]
            for key in extra:
                os.environ.pop(key, None)
        outs.append(h)
    for key in ("ref_idx", "codes", "scale", "zmin", "z"):
        for other in outs[1:]:
            assert np.array_equal(outs[0][key].view(np.uint8), other[key].view(np.uint8)), key


@pytest.mark.parametrize("cfg", [LLAMA8K.with_(name="llama_B3_T1500", B=3, T=1500), RAGGED[0],
                                 RAGGED[2], LLAMA8K.with_(name="llama_g64_B2_T1200", B=2, T=1200,
                                                          g=64),
                                 LLAMA8K.with_(name="llama_identity_T1200", T=1200, b=16)],
                         ids=lambda c: c.name)
def test_w3_tilings_bit_identical(cfg):
    """The W3 product with the quantiser runs 256 x 256 tiles, or 128 x 128
    tiles two to a CU where the wide ones would leave most CUs idle;
    RKV_W3_TILE forces either.  The tile shape changes no output's
    accumulation order, so records and z are the same bits: g = 8 to 64,
    INT2, INT4 and identity mode, d_c = 96 (a ragged column tile)."""
    outs = []
    for tiling in ("wide", "narrow"):
        os.environ["RKV_W3_TILE"] = tiling
        try:
            _, _, h, _ = P.run_encode(generate(cfg))
        finally:
            del os.environ["RKV_W3_TILE"]
        outs.append(h)
    for key in ("ref_idx", "codes", "scale", "zmin", "z"):
        assert np.array_equal(outs[0][key].view(np.uint8), outs[1][key].view(np.uint8)), key

def _bf16_bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


TIE_LAYOUTS = {
    # one chunk, one scan span: the displaced pair meets the run of ties
    "one_chunk": dict(T=1024, dup=(3, 5, 9, 12, 20, 21), close=30, probes=(250, 301, 517, 1001)),
    # duplicates in both halves of chunk 0 and in chunk 1 (192 references
    # per chunk): the two-list combine and the chunk merge see the ties
    "across_chunks": dict(T=2560, dup=(100, 150, 191, 192, 200, 250), close=300,
                          probes=(2405, 2466, 2559)),
}


@pytest.mark.parametrize("layout", list(TIE_LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_encode_exact_ties_keep_smaller_positions(dtype, layout):
    """Equal distances go to the smaller position ([RKV] §2.1, the (d, j)
    order).  Six references are one identical row, a later reference equals
    the probe tokens, and the probes sit near the duplicate row: each probe's
    distances to the six are exactly equal on both sides, and the later,
    closer reference arrives after four of them fill a list.  The kept set
    must be that reference and the three smallest duplicate positions, with
    no tie excused."""
    lay = TIE_LAYOUTS[layout]
    cfg = LLAMA8K.with_(name=f"ties_{dtype}_{layout}", B=1, T=lay["T"], N=2, D=32, d_ff=64,
                        d_c=64, k=4, g=32, b=4, stride=8, n_protos=8, dtype=dtype)
    w = generate(cfg)
    kv = w.kv_f32()[0].astype(np.float32)              # [T, C]
    s = cfg.stride
    dup = [s * m for m in lay["dup"]]                  # reference positions
    close, probes = s * lay["close"], list(lay["probes"])  # a later reference; non-references
    rng = np.random.default_rng(5)
    base = kv[dup[0]].copy()
    probe = base + 0.1 * np.abs(base).mean() * rng.standard_normal(cfg.C).astype(np.float32)
    rows = {t: base for t in dup}
    rows[close] = probe
    rows.update({t: probe for t in probes})
    for t, r in rows.items():
        kv[t] = r
    if dtype == "bf16":
        w.kv[0] = _bf16_bits(kv)
    else:
        w.kv[0] = kv
    _, _, h, _ = P.run_encode(w)
    kvb = w.kv_f32()[0].astype(np.float64)
    W1, W2, W3 = (x.astype(np.float64) for x in w.weights_f32())
    orc = O.encode_tokens(kvb, W1, W2, W3, np.array(probes), k=cfg.k, g=cfg.g, b=cfg.b, s=s)
    want = np.sort(np.array([close] + dup[:3]))
    for i, t in enumerate(probes):
        assert np.array_equal(np.sort(orc["ref_idx"][i]), want), (t, orc["ref_idx"][i])
        assert np.array_equal(h["ref_idx"][0, t], orc["ref_idx"][i]), (t, h["ref_idx"][0, t], want)
    # every other token: the usual bars
    P.compare_tokens(w, h, {0: np.arange(cfg.T)}, log=print)


@pytest.mark.parametrize("b,g", [(4, 32), (2, 32), (4, 8), (2, 16), (4, 64), (16, 32)])
def test_quantize_export_bit_exact(b, g):
    rng = np.random.default_rng(b * 100 + g)
    d_c = 128
    z = np.concatenate([
        rng.standard_normal((300, d_c)),
        rng.standard_t(2, size=(100, d_c)) * 1e-3,
        np.zeros((5, d_c)),                          # all-zero rows
        np.full((5, d_c), 0.1),                      # constant groups, not fp16-exact
        np.tile(np.arange(d_c) % g, (5, 1)) * 0.5,   # ramps with half-grid ties
    ]).astype(np.float32)
    z[7, :g] = 3.25                                  # one constant group inside a row
    p = R.params(B=1, T=1, N=1, D=32, d_ff=32, d_c=d_c, k=4, g=g, b=b, ref_stride=1, dtype="f32")
    zt = torch.from_numpy(z).cuda()
    codes = torch.empty((len(z), d_c * b // 8), dtype=torch.uint8, device="cuda")
    sc = torch.empty((len(z), d_c // g), dtype=torch.float16, device="cuda")
    zm = torch.empty_like(sc)
    R.rkv_quantize(p, zt, len(z), codes, sc, zm, torch.cuda.current_stream())
    torch.cuda.synchronize()
    q, dh, mh = O.quantize(z.astype(np.float64), g, b)
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(q, b))
    if b == O.IDENTITY_BITS:                         # no group numbers in identity mode
        return
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), dh.view(np.uint16))
    assert np.array_equal(zm.cpu().numpy().view(np.uint16), mh.view(np.uint16))


@pytest.mark.parametrize("b", [4, 2, 16])
def test_gather_bit_exact_f32_and_bf16(b):
    rng = np.random.default_rng(5 + b)
    B, T, d_c, g = 2, 300, 64, 32
    z = rng.standard_normal((B * T, d_c))
    z[::7] = 0.0
    q, dh, mh = O.quantize(z, g, b)
    codes = O.pack_codes(q, b)
    idx = np.concatenate([rng.integers(0, B * T, 500), [0, B * T - 1, -1, B * T, 10 ** 6, 3, 3]])
    idx = idx.astype(np.int32)
    p = R.params(B=B, T=T, N=1, D=32, d_ff=32, d_c=d_c, k=4, g=g, b=b, ref_stride=4, dtype="f32")
    dc = torch.from_numpy(codes).cuda()
    ds = torch.from_numpy(dh).cuda()
    dz = torch.from_numpy(mh).cuda()
    di = torch.from_numpy(idx).cuda()
    out32 = torch.empty((len(idx), d_c), dtype=torch.float32, device="cuda")
    out16 = torch.empty((len(idx), d_c), dtype=torch.bfloat16, device="cuda")
    st = torch.cuda.current_stream()
    R.rkv_dequant_gather(p, dc, ds, dz, di, len(idx), out32, "f32", st)
    R.rkv_dequant_gather(p, dc, ds, dz, di, len(idx), out16, "bf16", st)
    R.rkv_dequant_gather(p, dc, ds, dz, di, 0, out32, "f32", st)      # empty: no-op
    torch.cuda.synchronize()
    want = O.gather(codes, dh, mh, idx, g=g, b=b, d_c=d_c)
    got = out32.cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    g16 = P.bf16_bits_of(out16)
    assert np.array_equal(g16[~nan], P.expected_bf16(want)[~nan])
    assert np.all(np.isnan(out16.float().cpu().numpy()[nan]))
