"""Pins of the fp64 CPU oracle against what the ResidualKV notes and plain
mathematics fix ([RKV] = the ResidualKV reading notes, arXiv 2602.08005v2,
with the notes' own section numbers).

Each test checks the oracle against something other than itself: brute force
by another route, a closed-form identity, a special case with a known answer,
a library routine, or a number the notes print.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rkv_oracle as O
from synth import CONFIGS, generate
from synth.configs import LLAMA8K, MM_INT2, QWEN_LIKE, TINY

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    w = generate(TINY)
    kv = w.kv_f32()[0].astype(np.float64)
    W1, W2, W3 = (a.astype(np.float64) for a in w.weights_f32())
    return w, kv, W1, W2, W3


def _brute_topk(kv, t, s, k):
    """Pure-Python brute force: every earlier reference, sorted on (d, j) tuples."""
    x = [float(v) for v in kv[t]]
    cands = []
    for j in range(0, t, s):
        y = kv[j]
        d = 0.0
        for a, bb in zip(x, y):
            d += (a - float(bb)) ** 2
        cands.append((d, j))
    cands.sort()
    return [j for _, j in cands[:min(k, len(cands))]]


# ------------------------------------------------------------ selection
def test_selection_matches_pure_python_brute_force(tiny):
    w, kv, *_ = tiny
    s, k = TINY.stride, TINY.k
    for t in range(TINY.T):
        if t % s == 0:
            continue
        R, _ = O.retrieve(kv, t, s, k)
        assert sorted(R.tolist()) == sorted(_brute_topk(kv, t, s, k)), t


@pytest.mark.parametrize("cfg", [LLAMA8K, QWEN_LIKE, MM_INT2], ids=lambda c: c.name)
def test_selection_matches_sorted_brute_force_on_slices(cfg):
    """Wide shapes: full distance list by broadcasting, Python sort on tuples."""
    w = generate(cfg.with_(T=512, B=1, mm_blocks=1, mm_block_len=200))
    kv = w.kv_f32()[0].astype(np.float64)
    s, k = cfg.stride, cfg.k
    rng = np.random.default_rng(1)
    ts = [t for t in rng.choice(cfg.T if cfg.T <= 512 else 512, 60, replace=False) if t % s]
    for t in ts:
        refs = np.arange(0, t, s)
        d = ((kv[refs] - kv[t]) ** 2).sum(axis=1)
        want = [j for _, j in sorted(zip(d.tolist(), refs.tolist()))[:min(k, len(refs))]]
        R, _ = O.retrieve(kv, int(t), s, k)
        assert sorted(R.tolist()) == sorted(want)


def test_topk_minimises_retrieval_radius(tiny):
    """[RKV] §2.8: for a fixed pool and subset size, the k_i nearest
    references minimise rho_i^2.  Checked by enumerating every subset."""
    _, kv, *_ = tiny
    s, k = TINY.stride, TINY.k
    for t in [41, 77, 99, 130, 161, 189, 203, 222, 237, 255]:
        pool = np.arange(0, t, s)
        d = np.array([((kv[t] - kv[j]) ** 2).sum() for j in pool])
        best = min(d[list(c)].mean() for c in itertools.combinations(range(len(pool)), k))
        R, _ = O.retrieve(kv, t, s, k)
        rho2 = np.mean([((kv[t] - kv[j]) ** 2).sum() for j in R])
        assert rho2 == pytest.approx(best, rel=1e-12, abs=0)


def test_warmup_neighbour_count():
    """k_i = min(k, |T_ref,i|) ([RKV] §2.1); |T_ref,t| = ceil(t/s) with refs at t % s == 0."""
    rng = np.random.default_rng(3)
    for T, s, k in [(40, 8, 4), (37, 5, 3), (20, 3, 8), (9, 16, 4)]:
        kv = rng.standard_normal((T, 12))
        W1 = rng.standard_normal((12, 8)); W2 = rng.standard_normal((12, 8))
        W3 = rng.standard_normal((8, 8))
        out = O.encode_tokens(kv, W1, W2, W3, range(T), k=k, g=8, b=4, s=s)
        for t in range(T):
            n = int((out["ref_idx"][t] >= 0).sum())
            want = 0 if t % s == 0 else min(k, math.ceil(t / s))
            assert n == want, (T, s, k, t)
            got = out["ref_idx"][t][:n]
            assert np.all(got % s == 0) and np.all(got < t) and np.all(np.diff(got) > 0)


# ------------------------------------------------------------ mean (Theorem IV.1)
def test_theorem_iv1_decomposition(tiny):
    """rho_i^2 = ||Delta_i||^2 + V_i exactly ([RKV] §2.8, Theorem IV.1).
    A wrong mean (wrong divisor, wrong rows) breaks the identity."""
    _, kv, *_ = tiny
    s, k = TINY.stride, TINY.k
    for t in range(1, TINY.T):
        if t % s == 0:
            continue
        R, _ = O.retrieve(kv, t, s, k)
        m = O.reference_mean(kv, R)
        rho2 = np.mean([((kv[t] - kv[j]) ** 2).sum() for j in R])
        delta2 = ((kv[t] - m) ** 2).sum()
        V = np.mean([((kv[j] - m) ** 2).sum() for j in R])
        assert rho2 == pytest.approx(delta2 + V, rel=1e-12)


# ------------------------------------------------------------ compressor
def test_fc_matches_torch_fp64(tiny):
    _, kv, W1, W2, W3 = tiny
    x = kv[:50]
    want = (torch.nn.functional.silu(torch.from_numpy(x) @ torch.from_numpy(W1))
            * (torch.from_numpy(x) @ torch.from_numpy(W2))) @ torch.from_numpy(W3)
    np.testing.assert_allclose(O.f_c(x, W1, W2, W3), want.numpy(), rtol=1e-12, atol=1e-14)
    # square weights, so a transposed W1, W2 or W3 would still multiply
    rng = np.random.default_rng(5)
    Ws = [rng.standard_normal((16, 16)) / 4 for _ in range(3)]
    xs = rng.standard_normal((7, 16))
    t = [torch.from_numpy(a) for a in (xs, *Ws)]
    want = (torch.nn.functional.silu(t[0] @ t[1]) * (t[0] @ t[2])) @ t[3]
    np.testing.assert_allclose(O.f_c(xs, *Ws), want.numpy(), rtol=1e-12, atol=1e-14)


def test_z_is_zero_when_token_equals_its_references():
    rng = np.random.default_rng(5)
    T, s, C = 64, 8, 16
    kv = rng.standard_normal((T, C))
    v = rng.standard_normal(C)
    for j in (8, 16, 24, 32):
        kv[j] = v
    kv[45] = v
    W1 = rng.standard_normal((C, 24)); W2 = rng.standard_normal((C, 24))
    W3 = rng.standard_normal((24, 16))
    out = O.encode_tokens(kv, W1, W2, W3, [45], k=4, g=8, b=4, s=s)
    assert out["ref_idx"][0].tolist() == [8, 16, 24, 32]
    assert np.all(out["z"][0] == 0.0)
    assert np.all(out["codes"] == 0) and np.all(out["scale"] == 0) and np.all(out["zmin"] == 0)


def test_subtraction_after_encoding_is_not_encoding_the_difference(tiny):
    """[RKV] §2.3: f_c(kv) - f_c(mean) differs from f_c(kv - mean) (f_c is non-linear)."""
    _, kv, W1, W2, W3 = tiny
    s, k = TINY.stride, TINY.k
    for t in [50, 100, 150, 200, 250]:
        R, _ = O.retrieve(kv, t, s, k)
        m = O.reference_mean(kv, R)
        z = O.residual_latent(kv[t], m, W1, W2, W3)
        wrong = O.f_c(kv[t] - m, W1, W2, W3)
        assert np.linalg.norm(z - wrong) / np.linalg.norm(z) > 1e-2


def test_zero_gate_weights_give_zero_latent(tiny):
    _, kv, W1, W2, W3 = tiny
    out = O.encode_tokens(kv, W1, np.zeros_like(W2), W3, range(30, 60), k=4, g=32, b=4, s=8)
    assert np.all(out["z"] == 0.0)


def test_encode_all_equals_per_token(tiny):
    w, kv, W1, W2, W3 = tiny
    full = O.encode(kv[None], W1, W2, W3, k=4, g=32, b=4, s=8)
    some = O.encode_tokens(kv, W1, W2, W3, [3, 8, 9, 100, 255], k=4, g=32, b=4, s=8)
    for i, t in enumerate([3, 8, 9, 100, 255]):
        assert np.array_equal(full["ref_idx"][0, t], some["ref_idx"][i])
        assert np.array_equal(full["codes"][0, t], some["codes"][i])
        np.testing.assert_allclose(full["z"][0, t], some["z"][i], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ quantiser
def _read_kv(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def test_quantiser_ramp_golden():
    gd = _read_kv(os.path.join(GOLD, "quant_ramp_b4.txt"))
    z = np.arange(32, dtype=np.float64)[None, :]
    q, dh, mh = O.quantize(z, 32, 4)
    assert float(dh[0, 0]) == float(gd["delta_h"][0])
    assert float(mh[0, 0]) == float(gd["zmin_h"][0])
    assert q[0].tolist() == [int(v) for v in gd["codes"]]
    assert O.pack_codes(q, 4)[0].tolist() == [int(h, 16) for h in gd["packed_hex"]]
    deq = O.dequantize(q, dh, mh, 32)[0]
    assert deq.tolist() == [(i // 2) * 529 / 256 for i in range(32)]


def test_packing_golden():
    gd = _read_kv(os.path.join(GOLD, "packing.txt"))
    for b in (4, 2):
        q = np.array([[int(v) for v in gd[f"b{b}_codes"]]])
        packed = O.pack_codes(q, b)[0].tolist()
        assert packed == [int(h, 16) for h in gd[f"b{b}_hex"]]
        assert O.unpack_codes(O.pack_codes(q, b), b, q.shape[1]).tolist() == q.tolist()


@pytest.mark.parametrize("b", [2, 4])
def test_quantiser_on_grid_values_are_exact(b):
    """Values already on a grid m + q*Delta (Delta, m exact in fp16, both ends
    present) must come back with those very codes and decode exactly."""
    rng = np.random.default_rng(7)
    L = 2 ** b - 1
    for m, delta in [(-1.5, 0.25), (0.0, 1.0), (3.0, 0.0625), (-100.0, 8.0)]:
        q = rng.integers(0, L + 1, size=(20, 32))
        q[:, 0] = 0
        q[:, 1] = L
        z = m + q * delta
        qq, dh, mh = O.quantize(z, 32, b)
        assert np.array_equal(qq, q)
        assert np.all(dh.astype(np.float64) == delta) and np.all(mh.astype(np.float64) == m)
        assert np.array_equal(O.dequantize(qq, dh, mh, 32).astype(np.float64), z)


def test_quantiser_rounds_half_to_even():
    # group: 0 and 15 fix min = 0 and Delta = 1; midpoints k + 0.5 round to even
    z = np.array([[0.0, 15.0, 0.5, 1.5, 2.5, 3.5, 12.5, 13.5]])
    q, dh, mh = O.quantize(z, 8, 4)
    assert q[0].tolist() == [0, 15, 0, 2, 2, 4, 12, 14]


def test_constant_group_keeps_value_without_division():
    """[RKV] §2.4: a constant group is kept as its value (no divide by zero)."""
    z = np.zeros((3, 64))
    z[0, :32] = 0.375          # exact in fp16
    z[1, 32:] = -7.25          # exact in fp16
    z[2, :32] = 0.1            # not exact in fp16: kept as fp16(0.1)
    q, dh, mh = O.quantize(z, 32, 4)
    assert np.all(q == 0) and np.all(dh == 0)
    deq = O.dequantize(q, dh, mh, 32)
    assert np.all(deq[0, :32] == 0.375) and np.all(deq[0, 32:] == 0.0)
    assert np.all(deq[1, 32:] == -7.25)
    assert np.all(deq[2, :32] == np.float32(np.float16(0.1)))
    zero = O.encode_tokens(np.zeros((20, 8)), np.ones((8, 8)), np.ones((8, 8)),
                           np.ones((8, 32)), range(20), k=4, g=32, b=4, s=4)
    assert np.all(zero["codes"] == 0) and np.all(zero["scale"] == 0) and np.all(zero["zmin"] == 0)


@pytest.mark.parametrize("b", [2, 4])
def test_quantiser_error_bounds(b):
    """Per coordinate |z~ - z| <= Delta_h/2 plus the slack of storing Delta and
    z_min in fp16; and the norm bound of [RKV] §2.8 (Theorem IV.1, quantisation
    part): ||e_q|| <= sqrt(sum |G| range^2) / (2(2^b-1)) <= sqrt(g/2)/(2^b-1) ||z||,
    with the same fp16 slack added."""
    rng = np.random.default_rng(11)
    g, L = 32, 2 ** b - 1
    z = np.concatenate([rng.standard_normal((200, 128)),
                        0.01 * rng.standard_t(3, size=(200, 128)),
                        rng.uniform(-50, 50, size=(200, 128))])
    q, dh, mh = O.quantize(z, g, b)
    assert q.min() >= 0 and q.max() <= L
    deq = O.dequantize(q, dh, mh, g).astype(np.float64)
    zf = z.astype(np.float32).astype(np.float64)
    err_norm2 = np.zeros(len(z))
    bound2 = np.zeros(len(z))
    for gi, (a, e) in enumerate(O.group_bounds(128, g)):
        zg = zf[:, a:e]
        lo, hi = zg.min(1), zg.max(1)
        delta = (hi - lo) / L
        d16 = dh[:, gi].astype(np.float64)
        m16 = mh[:, gi].astype(np.float64)
        slack = np.abs(m16 - lo) + L * np.abs(d16 - delta) + 1e-6 * (np.abs(hi) + np.abs(lo))
        per = d16 / 2 + slack
        err = np.abs(deq[:, a:e] - zg)
        assert np.all(err <= per[:, None]), gi
        err_norm2 += (err ** 2).sum(1)
        bound2 += (e - a) * ((hi - lo) / (2 * L) + slack) ** 2
    assert np.all(np.sqrt(err_norm2) <= np.sqrt(bound2))
    # second inequality (range^2 <= 2||z_G||^2), data side only
    exact2 = sum((e - a) * (zf[:, a:e].max(1) - zf[:, a:e].min(1)) ** 2
                 for a, e in O.group_bounds(128, g))
    assert np.all(np.sqrt(exact2) / (2 * L) <= math.sqrt(g / 2) / L * np.linalg.norm(zf, axis=1) + 1e-12)


def test_quantiser_codes_use_the_stored_fp16_grid():
    """[RKV] §2.4 with reading: codes against the stored Delta_h and m_h.
    tests/golden/quant_stored_grid.txt derives by hand a group whose fp16
    minimum moves off min and one whose fp16 step moves off Delta; against the
    unrounded numbers four codes of each group would differ."""
    gd = _read_kv(os.path.join(GOLD, "quant_stored_grid.txt"))
    z = np.array([[int(v) / 4096.0 for v in gd["z_num_4096"]]])
    q, dh, mh = O.quantize(z, 8, 4)
    assert dh[0].astype(np.float64).tolist() == [float(v) for v in gd["delta_h"]]
    assert mh[0].astype(np.float64).tolist() == [float(v) for v in gd["zmin_h"]]
    assert q[0].tolist() == [int(v) for v in gd["codes"]]
    deq = O.dequantize(q, dh, mh, 8)[0].astype(np.float64)
    want = [float(mh[0, j // 8]) + q[0, j] * float(dh[0, j // 8]) for j in range(16)]
    assert deq.tolist() == want


def test_quantiser_decides_codes_on_the_float32_latent():
    """Reading: the integer decision is taken in float32.  The group
    {0, 15} fixes Delta_h = 1, m_h = 0.  3.5 - 2^-30 lies below the half-way
    point in float64 (code 3), but float32 has spacing 2^-22 near 3.5, so the
    latent rounds to 3.5 and half-to-even gives code 4; 5.5 + 2^-30 rounds to
    5.5 and gives 6 (float64: 6 as well); 6.5 - 2^-30 gives 6 either way."""
    z = np.array([[0.0, 15.0, 3.5 - 2.0 ** -30, 5.5 + 2.0 ** -30, 6.5 - 2.0 ** -30,
                   1.0, 2.0, 3.0]])
    q, dh, mh = O.quantize(z, 8, 4)
    assert float(dh[0, 0]) == 1.0 and float(mh[0, 0]) == 0.0
    assert q[0].tolist() == [0, 15, 4, 6, 6, 1, 2, 3]


def test_short_last_group():
    z = np.arange(40, dtype=np.float64)[None, :]   # groups [0,32) and [32,40)
    q, dh, mh = O.quantize(z, 32, 4)
    assert dh.shape == (1, 2)
    assert float(mh[0, 1]) == 32.0 and float(dh[0, 1]) == float(np.float16(np.float32(7) / np.float32(15)))


# ------------------------------------------------------------ gather
def test_gather_is_dequantise_of_selected_rows_and_nan_out_of_range():
    rng = np.random.default_rng(13)
    z = rng.standard_normal((10, 64))
    q, dh, mh = O.quantize(z, 32, 4)
    codes = O.pack_codes(q, 4)
    idx = np.array([3, 0, 9, 3, -1, 10])
    out = O.gather(codes, dh, mh, idx, g=32, b=4, d_c=64)
    deq = O.dequantize(q, dh, mh, 32)
    assert np.array_equal(out[0], deq[3]) and np.array_equal(out[1], deq[0])
    assert np.array_equal(out[2], deq[9]) and np.array_equal(out[3], deq[3])
    assert np.all(np.isnan(out[4])) and np.all(np.isnan(out[5]))
    assert O.gather(codes, dh, mh, np.array([], dtype=np.int64), g=32, b=4, d_c=64).shape == (0, 64)


# ------------------------------------------------------------ storage accounting
def test_storage_accounting_matches_printed_numbers():
    gd = json.load(open(os.path.join(GOLD, "storage_accounting.json")))
    assert O.q_b(4) == gd["q4"] and O.q_b(2) == gd["q2"]
    for key in ("kr_example", "kr_example_4_full_layers"):
        e = gd[key]
        kr = O.keep_ratio(e["beta"], e["rho_ref"], e["q_b"], e["dc_over_2dk"])
        assert round(100 * kr, e["printed_decimals"]) == e["printed_percent"]
    # one record per non-reference token: b-bit codes + two fp16 per group
    for C, d_c, b in [(2048, 512, 4), (2048, 512, 2), (1024, 256, 4), (64, 32, 4)]:
        assert O.storage_ratio_vs_fp16(C, d_c, 32, b) == pytest.approx(O.q_b(b) * d_c / C, rel=1e-15)


# ------------------------------------------------------------ generators
def test_generators_are_deterministic_and_shaped():
    a = generate(TINY)
    b = generate(TINY)
    assert np.array_equal(a.kv, b.kv) and np.array_equal(a.w3, b.w3)
    assert a.kv.shape == (1, 256, 64) and a.kv.dtype == np.float32
    c = generate(LLAMA8K.with_(T=64))
    assert c.kv.dtype == np.uint16 and c.kv.shape == (1, 64, 2048)
    m = generate(MM_INT2.with_(B=2, T=4096))
    for segs in m.segments:
        assert segs[0][1] == 0 and segs[-1][2] == 4096
        assert all(x[2] == y[1] for x, y in zip(segs, segs[1:]))
    full = [s for s in generate(MM_INT2.with_(B=1)).segments[0] if s[0] == "image"]
    assert len(full) == 24 and all(e - a_ == 576 for _, a_, e in full)


def test_equal_distances_prefer_the_earlier_reference():
    """Ties in distance are broken by the smaller position (a reading: the notes
    leave ties open); copies of one vector at two reference slots must pick the
    earlier slot first."""
    rng = np.random.default_rng(17)
    T, s, C = 80, 8, 16
    kv = rng.standard_normal((T, C)) * 5
    v = rng.standard_normal(C)
    kv[40] = v
    kv[16] = v
    kv[64] = v
    kv[71] = v + 1e-3
    for k, want in [(1, [16]), (2, [16, 40]), (3, [16, 40, 64])]:
        R, _ = O.retrieve(kv, 71, s, k)
        assert R.tolist() == want


def test_zero_references_reduce_z_to_library_compressor():
    """With every reference equal to the zero vector the mean is 0 and
    f_c(0) = 0 (no biases), so z must equal f_c(kv_t) computed by torch."""
    rng = np.random.default_rng(19)
    T, s, C = 48, 6, 16
    kv = rng.standard_normal((T, C))
    kv[::s] = 0.0
    W1 = rng.standard_normal((C, 24)); W2 = rng.standard_normal((C, 24))
    W3 = rng.standard_normal((24, 32))
    ts = [t for t in range(T) if t % s]
    out = O.encode_tokens(kv, W1, W2, W3, ts, k=4, g=32, b=4, s=s)
    x = torch.from_numpy(kv[ts])
    want = (torch.nn.functional.silu(x @ torch.from_numpy(W1)) * (x @ torch.from_numpy(W2))) @ torch.from_numpy(W3)
    np.testing.assert_allclose(out["z"], want.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ restore
def _rope_gold():
    vals = {}
    with open(os.path.join(GOLD, "rope_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *rest = line.split()
            vals[key] = [float(v) for v in rest]
    return vals


def test_rope_matches_hand_worked_example():
    """[RKV] §2.1 note; values worked by hand in tests/golden/rope_example.txt."""
    g = _rope_gold()
    y = O.apply_rope(np.array(g["x"]), int(g["position"][0]), 1, int(g["D"][0]), g["theta"][0])
    np.testing.assert_allclose(y, g["y"], rtol=0, atol=1e-15)


def test_rope_position_zero_and_disabled_are_identity():
    x = np.random.default_rng(3).standard_normal(2 * 16)
    np.testing.assert_array_equal(O.apply_rope(x, 0, 2, 16, 10000.0), x)
    np.testing.assert_array_equal(O.apply_rope(x, 77, 2, 16, 0.0), x)


def test_rope_preserves_pair_norms_and_relative_positions():
    """A rotation keeps each (d, d + D/2) pair's length, and the score of two
    rotated vectors depends only on their position difference."""
    rng = np.random.default_rng(4)
    N, D, th = 2, 16, 500000.0
    q, k = rng.standard_normal(N * D), rng.standard_normal(N * D)
    rq = O.apply_rope(q, 1234, N, D, th).reshape(N, D)
    qq = q.reshape(N, D)
    np.testing.assert_allclose(rq[:, :D // 2] ** 2 + rq[:, D // 2:] ** 2,
                               qq[:, :D // 2] ** 2 + qq[:, D // 2:] ** 2, rtol=1e-12)
    s1 = O.apply_rope(q, 900, N, D, th) @ O.apply_rope(k, 250, N, D, th)
    s2 = O.apply_rope(q, 1650, N, D, th) @ O.apply_rope(k, 1000, N, D, th)
    assert abs(s1 - s2) < 1e-9 * (1 + abs(s1))


@pytest.fixture(scope="module")
def tiny_encoded(tiny):
    w, kv, W1, W2, W3 = tiny
    c = TINY
    enc = O.encode(kv[None], W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride)
    return enc


def _restore(enc, kv, Wd, idx, theta):
    c = TINY
    flat = lambda a: a.reshape(-1, *a.shape[2:])
    return O.restore(flat(enc["codes"]), flat(enc["scale"]), flat(enc["zmin"]), flat(enc["ref_idx"]),
                     kv[None], Wd, np.asarray(idx), s=c.stride, N=c.N, D=c.D, g=c.g, b=c.b,
                     d_c=c.d_c, rope_theta=theta)


def test_restore_reference_tokens_are_their_stored_rows(tiny, tiny_encoded):
    """[RKV] §2.4/§2.5: references are stored as they are; only their keys are rotated."""
    w, kv, *_ = tiny
    Wd = np.random.default_rng(5).standard_normal((TINY.d_c, TINY.C))
    refs = np.arange(0, TINY.T, TINY.stride)
    out = _restore(tiny_encoded, kv, Wd, refs, 0.0)
    np.testing.assert_array_equal(out, kv[refs])
    out_r = _restore(tiny_encoded, kv, Wd, refs, 10000.0)
    nd = TINY.N * TINY.D
    for n, t in enumerate(refs):
        np.testing.assert_allclose(out_r[n, :nd], O.apply_rope(kv[t, :nd], t, TINY.N, TINY.D, 10000.0))
        np.testing.assert_array_equal(out_r[n, nd:], kv[t, nd:])


def test_restore_of_a_zero_record_or_zero_decoder_is_the_reference_mean(tiny, tiny_encoded):
    """f_d(0) = 0 and a zero W_d leave exactly the mean of the stored references ([RKV] §2.5)."""
    w, kv, *_ = tiny
    enc = {k: v.copy() for k, v in tiny_encoded.items()}
    t = 37
    enc["codes"][0, t] = 0
    enc["scale"][0, t] = 0
    enc["zmin"][0, t] = 0
    Wd = np.random.default_rng(6).standard_normal((TINY.d_c, TINY.C))
    R = [int(p) for p in tiny_encoded["ref_idx"][0, t] if p >= 0]
    mean = kv[R].mean(axis=0)
    np.testing.assert_allclose(_restore(enc, kv, Wd, [t], 0.0)[0], mean, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(_restore(tiny_encoded, kv, np.zeros_like(Wd), [t], 0.0)[0], mean,
                               rtol=1e-15, atol=1e-15)


def test_restore_with_an_identity_decoder_returns_the_token_within_the_quantiser_bound():
    """With d_c = 2 d_k, W_d = I and records that quantise kv_t - mean, the
    restore is kv_t up to the quantiser's error: at most Delta_h / 2 plus the
    fp16 slack of the record per coordinate ([RKV] §2.4, §2.5)."""
    c = TINY.with_(d_c=TINY.C)
    rng = np.random.default_rng(8)
    kv = rng.standard_normal((1, 40, c.C))
    t = 21
    pos = O.candidate_pool(t, c.stride)
    R, _ = O.retrieve(kv[0], t, c.stride, c.k)
    mean = O.reference_mean(kv[0], R)
    q, dh, mh = O.quantize((kv[0, t] - mean)[None].astype(np.float32), c.g, c.b)
    codes = np.zeros((40, c.d_c * c.b // 8), np.uint8)
    scale = np.zeros((40, c.d_c // c.g), np.float16)
    zmin = np.zeros_like(scale)
    codes[t] = O.pack_codes(q, c.b)[0]
    scale[t], zmin[t] = dh[0], mh[0]
    ref_idx = np.full((40, c.k), -1, np.int64)
    ref_idx[t, :len(R)] = np.sort(R)
    out = O.restore(codes, scale, zmin, ref_idx, kv, np.eye(c.C), np.array([t]), s=c.stride,
                    N=c.N, D=c.D, g=c.g, b=c.b, d_c=c.d_c, rope_theta=0.0)[0]
    step = np.repeat(dh[0].astype(np.float64), c.g)
    assert np.all(np.abs(out - kv[0, t]) <= step / 2 + 1e-3 * step + 1e-6)


def test_restore_out_of_range_rows_are_nan(tiny, tiny_encoded):
    w, kv, *_ = tiny
    Wd = np.zeros((TINY.d_c, TINY.C))
    out = _restore(tiny_encoded, kv, Wd, [-1, TINY.T, 5], 0.0)
    assert np.isnan(out[0]).all() and np.isnan(out[1]).all() and not np.isnan(out[2]).any()


# ------------------------------------------------------------------ schedule
def test_reference_schedule_reproduces_table_vi_counts():
    """[RKV] §4.6 Table VI, numbers printed by the notes (reading of T in the file)."""
    with open(os.path.join(GOLD, "reference_counts.json")) as f:
        g = json.load(f)
    got = [len(O.reference_schedule(g["T"], g["s0"], a, g["n_sink"])) for a in g["alpha"]]
    assert got == g["count"]


@pytest.mark.parametrize("ns", [4, 1000])
@pytest.mark.parametrize("alpha", [0.001, 0.02, 0.05, 0.1])
def test_reference_count_follows_the_logarithmic_approximation(alpha, ns):
    """[RKV] §2.6: ignoring the floor, N_ref(T) ~ log_{1+a}(1 + a (T - n_sink) / s0)
    references after the sinks.  The floor only shortens gaps, so the exact
    count is at least the approximation, and close to it.  A thousand sinks
    make the n_sink offset inside the floor visible in the count."""
    T, s0 = 262144, 10
    n = len(O.reference_schedule(T, s0, alpha, ns)) - ns
    approx = math.log1p(alpha * (T - ns) / s0) / math.log1p(alpha)
    assert approx <= n <= 1.02 * approx + 2


def test_dynamic_schedule_with_sinks_matches_hand_derivation():
    """[RKV] §2.6 recurrence with n_sink = 1000, alpha = 0.02, s0 = 10: the
    first sixteen positions after the sinks, derived by hand in
    tests/golden/dynamic_schedule_sinks.txt (the gap grows with p - n_sink)."""
    gd = _read_kv(os.path.join(GOLD, "dynamic_schedule_sinks.txt"))
    ns, alpha, s0 = int(gd["n_sink"][0]), float(gd["alpha"][0]), int(gd["s0"][0])
    want = [int(v) for v in gd["after_sinks"]]
    r = O.reference_schedule(want[-1] + 1, s0, alpha, ns)
    assert r[:ns].tolist() == list(range(ns))
    assert r[ns:].tolist() == want


def test_reference_schedule_special_cases():
    """alpha = 0 without sinks is the fixed stride; sinks come first and the
    recurrence starts right after them; gaps never shrink."""
    np.testing.assert_array_equal(O.reference_schedule(1000, 16), np.arange(0, 1000, 16))
    r = O.reference_schedule(5000, 10, 0.01, 4)
    assert list(r[:5]) == [0, 1, 2, 3, 4] and r[5] == 4 + 10
    gaps = np.diff(r[4:])
    assert np.all(np.diff(gaps) >= 0) and gaps[0] == 10


def test_dynamic_schedule_pool_and_selection_follow_the_schedule():
    """Under a dynamic schedule the pool of t is the scheduled references
    before t, and the encode's selections match brute force over that pool."""
    rng = np.random.default_rng(21)
    T, C = 160, 16
    kv = rng.standard_normal((T, C))
    refs = O.reference_schedule(T, 6, 0.05, 3)
    W1, W2 = rng.standard_normal((C, 8)), rng.standard_normal((C, 8))
    W3 = rng.standard_normal((8, 8))
    pos = [t for t in range(T) if t not in set(refs.tolist())]
    enc = O.encode_tokens(kv, W1, W2, W3, pos, k=3, g=8, b=4, s=6, alpha=0.05, n_sink=3)
    for i, t in enumerate(pos):
        pool = [int(p) for p in refs if p < t]
        d = [(float(((kv[t] - kv[p]) ** 2).sum()), p) for p in pool]
        want = sorted(p for _, p in sorted(d)[:min(3, len(pool))])
        got = [int(p) for p in enc["ref_idx"][i] if p >= 0]
        assert got == want, t


# ------------------------------------------------------------ append

def _append_all(kv, W1, W2, W3, *, k, g, b, s, alpha=0.0, n_sink=0):
    """Append every position in order to a cache whose rows start as NaN."""
    T = len(kv)
    cache = np.full_like(kv, np.nan)
    recs = []
    for t in range(T):
        r = O.append_token(cache, kv[t], t, W1, W2, W3, k=k, g=g, b=b, s=s, alpha=alpha,
                           n_sink=n_sink)
        if r["stored"]:
            cache[t] = kv[t]
        recs.append(r)
    return cache, recs


@pytest.mark.parametrize("alpha,n_sink", [(0.0, 0), (0.02, 2)])
def test_append_in_order_reproduces_the_prefix_encode(tiny, alpha, n_sink):
    """[RKV] §2.7 decode step 4: appending a sequence token by token to a cache
    that holds nothing but the stored references gives the records of encoding
    the whole prefix; rows that are never stored stay NaN and are never read
    (a NaN there would poison every distance)."""
    w, kv, W1, W2, W3 = tiny
    c = TINY
    cache, recs = _append_all(kv, W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride, alpha=alpha,
                              n_sink=n_sink)
    enc = O.encode(kv[None], W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride, alpha=alpha,
                   n_sink=n_sink)
    refs = O.reference_schedule(c.T, c.stride, alpha, n_sink)
    mask = np.zeros(c.T, bool)
    mask[refs] = True
    np.testing.assert_array_equal(cache[mask], kv[mask])
    assert np.isnan(cache[~mask]).all()
    for t, r in enumerate(recs):
        assert r["stored"] == mask[t]
        np.testing.assert_array_equal(r["ref_idx"], enc["ref_idx"][0, t])
        np.testing.assert_array_equal(r["codes"], enc["codes"][0, t])
        np.testing.assert_array_equal(r["scale"], enc["scale"][0, t])
        np.testing.assert_array_equal(r["zmin"], enc["zmin"][0, t])
        np.testing.assert_allclose(r["z"], enc["z"][0, t], rtol=0, atol=1e-12)


def test_append_selection_minimises_the_retrieval_radius():
    """[RKV] §2.8: the appended token's chosen set minimises the mean squared
    distance rho^2 to the chosen references over every k-subset of the pool
    (brute-force enumeration)."""
    rng = np.random.default_rng(31)
    T, C, s, k = 60, 12, 5, 3
    kv = rng.standard_normal((T, C))
    W = rng.standard_normal((C, 4))
    W3 = rng.standard_normal((4, 8))
    cache = np.full_like(kv, np.nan)
    cache[::s] = kv[::s]
    for t in (7, 23, 59):
        r = O.append_token(cache, kv[t], t, W, W, W3, k=k, g=8, b=4, s=s)
        pool = list(range(0, t, s))
        rho = lambda R: np.mean([((kv[t] - kv[j]) ** 2).sum() for j in R])
        best = min(rho(R) for R in itertools.combinations(pool, min(k, len(pool))))
        assert abs(rho([int(j) for j in r["ref_idx"] if j >= 0]) - best) <= 1e-12 * best


def test_append_of_a_reference_position_is_stored_with_a_zero_record(tiny):
    """[RKV] §2.4 and §2.7 step 4: a token the schedule makes a reference is stored as it is."""
    w, kv, W1, W2, W3 = tiny
    c = TINY
    cache = np.full_like(kv, np.nan)
    r = O.append_token(cache, kv[3 * c.stride], 3 * c.stride, W1, W2, W3, k=c.k, g=c.g, b=c.b,
                       s=c.stride)
    assert r["stored"]
    assert np.all(r["ref_idx"] == -1) and not r["codes"].any()
    assert not r["scale"].any() and not r["zmin"].any() and not r["z"].any()


# ------------------------------------------------------------ identity mode

def test_identity_mode_rounds_the_float32_latent_to_fp16():
    """Reading: in identity mode the stored fp16 value is rounded from the
    latent's float32 value.  1 + 2^-11 + 2^-40 lies just above the half-way
    point between the fp16 values 1 and 1 + 2^-10, but float32 (spacing
    2^-23 there) drops the 2^-40, leaving an exact tie that goes to the even
    value 1.0 (bits 0x3c00); 1 + 3*2^-11 rounds up to 1 + 2^-9 (0x3c02)
    either way."""
    z = np.array([[1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 3 * 2.0 ** -11]])
    q, _, _ = O.quantize(z, 32, 16)
    assert q[0].tolist() == [0x3C00, 0x3C02]


def test_identity_mode_stores_the_latent_as_fp16():
    """[RKV] §2.4: with quantisation off Q is the identity; the record is the
    latent in fp16 (2 bytes per coordinate, no group numbers), so z~ is z
    within half an fp16 ulp, and exactly z when z is an fp16 value."""
    rng = np.random.default_rng(8)
    z = rng.standard_normal((50, 64)) * np.exp(rng.uniform(-6, 3, (50, 1)))
    q, dh, mh = O.quantize(z, 32, 16)
    codes = O.pack_codes(q, 16)
    assert codes.shape == (50, 128) and not dh.any() and not mh.any()
    assert O.record_bytes_per_token(64, 32, 16) == 128
    back = O.dequantize(O.unpack_codes(codes, 16, 64), dh, mh, 32, 16).astype(np.float64)
    z32 = z.astype(np.float32).astype(np.float64)
    # fp16 normal range: |error| <= 2^-11 |z| (half an ulp, relative)
    normal = np.abs(z32) >= 2.0 ** -14
    assert np.all(np.abs(back - z32)[normal] <= 2.0 ** -11 * np.abs(z32)[normal])
    assert np.all(np.abs(back - z32)[~normal] <= 2.0 ** -25)
    exact = np.array([[0.0, 1.0, -2.5, 0.099975586, 65504.0, -6.1035156e-05, 3.0, 0.5]])
    qe, dhe, mhe = O.quantize(exact, 8, 16)
    np.testing.assert_array_equal(O.dequantize(qe, dhe, mhe, 8, 16), exact.astype(np.float32))
    # byte order: little-endian fp16 bits (1.0 = 0x3C00 -> 00 3C)
    assert O.pack_codes(O.quantize(np.array([[1.0]]), 1, 16)[0], 16).tolist() == [[0x00, 0x3C]]


# ------------------------------------------------------------ FP8 references

def test_fp8_storage_matches_hand_derived_values():
    """Every line of tests/golden/fp8_e4m3.txt was derived by hand from the format."""
    rows = []
    with open(os.path.join(GOLD, "fp8_e4m3.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                x, v, byte = line.split()[:3]
                rows.append((float(x), float(v), int(byte, 16)))
    x = np.array([r[0] for r in rows])
    np.testing.assert_array_equal(O.fp8_e4m3(x), [r[1] for r in rows])
    assert O.fp8_e4m3_bits(x).tolist() == [r[2] for r in rows]


def test_fp8_storage_matches_the_library_cast_and_round_trips():
    """torch's float8_e4m3fn cast (round to nearest even) agrees wherever it
    does not overflow (|x| <= 464); every finite byte decodes and re-encodes
    to itself."""
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000)),
                        np.ldexp(np.arange(-16, 17) / 16.0 + 1.0, rng.integers(-10, 8, 33))])
    x = x.astype(np.float32).astype(np.float64)
    x = x[np.abs(x) <= 464.0]
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.fp8_e4m3(x), lib)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.fp8_e4m3_value(finite)
    assert O.fp8_e4m3_bits(vals).tolist() == finite.tolist()
    assert np.abs(vals).max() == 448.0


def test_fp8_references_select_by_their_stored_values(tiny):
    """[RKV] §2.5: the encoder uses the references as stored.  With FP8
    references the selection is brute force over the FP8 values of the pool
    (rounded here by the library cast), and the mean is theirs."""
    w, kv, W1, W2, W3 = tiny
    c = TINY
    enc = O.encode_tokens(kv, W1, W2, W3, range(c.T), k=c.k, g=c.g, b=c.b, s=c.stride,
                          ref_fp8=True)
    kv8 = torch.from_numpy(kv.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    for t in range(1, c.T):
        if t % c.stride == 0:
            continue
        pool = list(range(0, t, c.stride))
        d = sorted((float(((kv[t] - kv8[j]) ** 2).sum()), j) for j in pool)
        want = sorted(j for _, j in d[:min(c.k, len(pool))])
        assert [int(j) for j in enc["ref_idx"][t] if j >= 0] == want, t
    t = 201
    mean8 = kv8[[int(j) for j in enc["ref_idx"][t] if j >= 0]].mean(axis=0)
    np.testing.assert_allclose(enc["z"][t], O.residual_latent(kv[t], mean8, W1, W2, W3),
                               rtol=0, atol=1e-12)


def test_fp8_append_in_order_reproduces_the_fp8_encode(tiny):
    """Appending token by token with FP8 references stores their FP8 values
    and reproduces the FP8-reference encode of the prefix."""
    w, kv, W1, W2, W3 = tiny
    c = TINY
    cache = np.full_like(kv, np.nan)
    enc = O.encode(kv[None], W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride, ref_fp8=True)
    for t in range(c.T):
        r = O.append_token(cache, kv[t], t, W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride,
                           ref_fp8=True)
        if r["stored"]:
            cache[t] = r["stored_row"]
        np.testing.assert_array_equal(r["codes"], enc["codes"][0, t])
        np.testing.assert_array_equal(r["ref_idx"], enc["ref_idx"][0, t])
    np.testing.assert_array_equal(cache[::c.stride], O.fp8_e4m3(kv[::c.stride]))


def test_fp8_restore_reads_the_stored_references(tiny):
    """[RKV] §2.5: the decoder adds the mean of the references as stored; a
    reference token restores to its FP8 stored row (unrotated), and a zero
    record restores to the mean of the FP8 rows."""
    w, kv, W1, W2, W3 = tiny
    c = TINY
    enc = O.encode(kv[None], W1, W2, W3, k=c.k, g=c.g, b=c.b, s=c.stride, ref_fp8=True)
    flat = lambda a: a.reshape(-1, *a.shape[2:])
    Wd = np.random.default_rng(9).standard_normal((c.d_c, c.C))
    refs = np.arange(0, c.T, c.stride)
    zero = np.zeros_like(flat(enc["codes"]))
    out = O.restore(zero, np.zeros_like(flat(enc["scale"])), np.zeros_like(flat(enc["zmin"])),
                    flat(enc["ref_idx"]), kv[None], Wd, np.array([*refs[:5], 201]), s=c.stride,
                    N=c.N, D=c.D, g=c.g, b=c.b, d_c=c.d_c, rope_theta=0.0, ref_fp8=True)
    np.testing.assert_array_equal(out[:5], O.fp8_e4m3(kv[refs[:5]]))
    R = [int(j) for j in enc["ref_idx"][0, 201] if j >= 0]
    np.testing.assert_allclose(out[5], O.fp8_e4m3(kv[R]).mean(axis=0), rtol=0, atol=1e-12)
