"""GPU parity of the decode-time append (rkv_append, [RKV] §2.7 decode step 4),
through the C ABI, against the fp64 oracle's encoding of the same positions
(the oracle's append_token is pinned to reproduce it token by token).

The cache's kv rows that are not references hold NaN, so a kernel that read
one would poison the result; records start as a byte pattern that rkv_append
must overwrite on appended rows and leave alone elsewhere.  The records are
compared with the same bars as the encode (rkv_parity).  Needs an MI355X."""
import numpy as np
import pytest
import torch

import reference_residual_encoding_amd as R
from synth import generate
from synth.configs import LLAMA8K, LLAMA8K_DYN, TINY, TINY_DYN

import rkv_parity as P

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _log(msg):
    print(msg, flush=True)


class Cache:
    """Device cache of one configuration: kv rows + records, in the
    layouts of include/rkv.h.  Non-reference kv rows hold NaN, and so do
    the reference rows unless prefill_refs.  With proj, the cache also keeps
    the references' projections (rkv_project_refs after the prefill) and
    appends through rkv_append_proj."""

    def __init__(self, w, prefill_refs: bool, device="cuda", proj: bool = False):
        cfg = self.cfg = w.cfg
        self.w = w
        self.p = P.params_of(cfg)
        n = cfg.B * cfg.T
        self.ref_mask = P.ref_mask_of(cfg)
        if cfg.ref_fp8:
            # the E4M3 store [B][nref][C]; 0x7F (NaN) where nothing is stored yet
            self.store_bytes = P.fp8_store(cfg, w.kv)
            kv = np.full_like(self.store_bytes, 0x7F)
            if prefill_refs:
                kv[:] = self.store_bytes
            self.expected_kv = kv
            self.kv = torch.from_numpy(kv.copy()).to(device)
        else:
            kv = np.array(w.kv, copy=True)
            nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)
            kv[:, ~self.ref_mask] = nan
            if not prefill_refs:
                kv[:, self.ref_mask] = nan
            self.expected_kv = kv                 # host copy of what the cache must hold
            self.kv = P.to_device(kv, cfg.dtype, device)
        self.w1, self.w2, self.w3 = (P.to_device(x, cfg.dtype, device) for x in (w.w1, w.w2, w.w3))
        u8 = lambda nbytes: torch.full((nbytes,), SENTINEL, dtype=torch.uint8, device=device)
        self.ref_idx = u8(n * cfg.k * 4).view(torch.int32).view(cfg.B, cfg.T, cfg.k)
        self.codes = u8(n * cfg.d_c * cfg.b // 8).view(cfg.B, cfg.T, -1)
        ng = 1 if cfg.b == 16 else cfg.d_c // cfg.g      # identity: no group numbers (not read)
        self.scale = u8(n * ng * 2).view(torch.float16).view(cfg.B, cfg.T, -1)
        self.zmin = u8(n * ng * 2).view(torch.float16).view(cfg.B, cfg.T, -1)
        self.z = u8(n * cfg.d_c * 4).view(torch.float32).view(cfg.B, cfg.T, cfg.d_c)
        self.proj = proj
        if proj:
            self.ws_bytes = R.rkv_append_proj_workspace_bytes(self.p)
            nbytes = R.rkv_ref_proj_bytes(self.p)
            assert nbytes == cfg.B * len(R.rkv_reference_positions(self.p)) * 2 * cfg.d_ff * 4
            self.ref_proj = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32,
                                       device=device)
        else:
            self.ws_bytes = R.rkv_append_workspace_bytes(self.p)
        assert self.ws_bytes > 0
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        if proj and prefill_refs:
            self.project()
        self.appended = np.zeros((cfg.B, cfg.T), bool)

    def project(self):
        """rkv_project_refs of the cache's stored references into ref_proj."""
        nbytes = R.rkv_project_refs_workspace_bytes(self.p)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=self.kv.device)
        R.rkv_project_refs(self.p, self.kv, self.w1, self.w2, self.ref_proj, ws, nbytes,
                           torch.cuda.current_stream())

    def append(self, pos):
        cfg = self.cfg
        pos = np.asarray(pos, dtype=np.int64)
        assert pos.shape == (cfg.B,)
        rows = np.zeros((cfg.B, cfg.C), dtype=self.w.kv.dtype)
        for b, t in enumerate(pos):
            if 0 <= t < cfg.T:
                rows[b] = self.w.kv[b, t]
                self.appended[b, t] = True
                if self.ref_mask[t] and cfg.ref_fp8:
                    j = int(np.cumsum(self.ref_mask)[t]) - 1
                    self.expected_kv[b, j] = self.store_bytes[b, j]
                elif self.ref_mask[t]:
                    self.expected_kv[b, t] = self.w.kv[b, t]
        kv_new = P.to_device(rows, cfg.dtype)
        d_pos = torch.from_numpy(pos.astype(np.int32)).cuda()
        if self.proj:
            R.rkv_append_proj(self.p, self.kv, self.ref_proj, kv_new, d_pos, self.w1, self.w2,
                              self.w3, self.ref_idx, self.codes, self.scale, self.zmin, self.z,
                              self.ws, self.ws_bytes, torch.cuda.current_stream())
        else:
            R.rkv_append(self.p, self.kv, kv_new, d_pos, self.w1, self.w2, self.w3, self.ref_idx,
                         self.codes, self.scale, self.zmin, self.z, self.ws, self.ws_bytes,
                         torch.cuda.current_stream())

    def check(self, name):
        """Parity of every appended row; untouched records keep the pattern;
        the cache holds exactly the appended (and prefilled) references."""
        cfg = self.cfg
        torch.cuda.synchronize()
        h = dict(ref_idx=self.ref_idx.cpu().numpy(), codes=self.codes.cpu().numpy(),
                 scale=self.scale.cpu().numpy(), zmin=self.zmin.cpu().numpy(),
                 z=self.z.cpu().numpy())
        pos = {b: np.flatnonzero(self.appended[b]) for b in range(cfg.B)}
        summary = P.compare_tokens(self.w, h, {b: v for b, v in pos.items() if v.size}, log=_log)
        untouched = ~self.appended
        assert (h["codes"][untouched] == SENTINEL).all(), f"{name}: a record outside the appended rows changed"
        assert (h["ref_idx"].view(np.uint8).reshape(cfg.B, cfg.T, -1)[untouched] == SENTINEL).all()
        assert (h["scale"].view(np.uint8).reshape(cfg.B, cfg.T, -1)[untouched] == SENTINEL).all()
        kv = self.kv.cpu()
        if cfg.ref_fp8:
            kv = kv.numpy()
        else:
            kv = kv.view(torch.int16).numpy().view(np.uint16) if cfg.dtype == "bf16" else kv.numpy()
        assert np.array_equal(kv.view(np.uint8), self.expected_kv.view(np.uint8)), \
            f"{name}: the cache's kv rows differ from the appended references"
        return summary


def _make(cfg, prefill, proj=False):
    return Cache(generate(cfg), prefill, proj=proj)


PROJ = pytest.mark.parametrize("proj", [False, True], ids=["append", "append_proj"])


@pytest.mark.parametrize("cfg", [TINY, TINY_DYN,
                                 TINY_DYN.with_(name="tiny_f32_dynamic_fp8ref", ref_fp8=True)],
                         ids=lambda c: c.name)
@PROJ
def test_append_every_position_in_order(cfg, proj):
    """An empty cache (all NaN) filled token by token reaches the same records
    as the oracle's encode of the prefix; reference rows land in the cache
    (with proj, so do their projections, which the later tokens' means
    read)."""
    _log(f"[case] append {cfg.name} in order proj={proj}")
    c = _make(cfg, prefill=False, proj=proj)
    for t in range(cfg.T):
        c.append(np.full(cfg.B, t))
    c.check(cfg.name)


RAGGED_BF16 = LLAMA8K.with_(name="append_ragged_bf16_b2_k5", B=3, T=1000, N=2, D=32, d_ff=96,
                            d_c=64, k=5, g=16, b=2, stride=7, n_protos=24)
RAGGED_F32 = LLAMA8K.with_(name="append_ragged_f32_k8_g64", B=2, T=700, N=1, D=64, d_ff=64,
                           d_c=128, k=8, g=64, b=4, stride=3, dtype="f32", n_protos=12, noise=0.3)


# C = 1280 rows of W1 | W2 in two slices (chunks 0 and 2, and chunk 1; the
# last chunk half past C) and d_ff = 4352 features, past the 4096 that the W3
# launch holds in LDS at a time
WIDE_FF = LLAMA8K.with_(name="append_c1280_dff4352_two_slices", B=2, T=600, N=5, D=128,
                        d_ff=4352, d_c=64, k=3, g=16, b=4, stride=5, n_protos=16)


@pytest.mark.parametrize("cfg", [RAGGED_BF16, RAGGED_F32,
                                 RAGGED_BF16.with_(name="append_ragged_bf16_identity", b=16),
                                 RAGGED_BF16.with_(name="append_ragged_bf16_fp8ref", ref_fp8=True),
                                 WIDE_FF],
                         ids=lambda c: c.name)
@PROJ
def test_append_independent_positions_per_sequence(cfg, proj):
    """Continuous batching: every call appends a different position in each
    sequence, in random order, with some sequences skipped (pos -1 or T)."""
    _log(f"[case] append {cfg.name} random positions proj={proj}")
    c = _make(cfg, prefill=True, proj=proj)
    rng = np.random.default_rng(17)
    perms = [rng.permutation(cfg.T) for _ in range(cfg.B)]
    for i in range(60):
        pos = np.array([perms[b][i] for b in range(cfg.B)])
        if i % 7 == 3:
            pos[i % cfg.B] = -1
        if i % 11 == 5:
            pos[(i + 1) % cfg.B] = cfg.T
        c.append(pos)
    c.check(cfg.name)


@pytest.mark.parametrize("cfg", [LLAMA8K.with_(B=2), LLAMA8K_DYN,
                                 LLAMA8K.with_(name="llama8b_T8k_fp8ref", B=2, ref_fp8=True)],
                         ids=lambda c: c.name)
@PROJ
def test_append_full_size_sampled(cfg, proj):
    """The Llama layer shape at 8k context: sampled positions (warm-up, tail,
    random), one per sequence per call."""
    _log(f"[case] append {cfg.name} sampled proj={proj}")
    c = _make(cfg, prefill=True, proj=proj)
    pos = [P.sample_positions(cfg.T, cfg.stride, 150, seed=40 + b, cfg=cfg) for b in range(cfg.B)]
    n = min(len(p) for p in pos)
    for i in range(n):
        c.append(np.array([pos[b][i] for b in range(cfg.B)]))
    c.check(cfg.name)


@PROJ
def test_append_bench_shape(proj):
    """The benchmark's append launch: 16 sequences at the end of a 32k
    context (pool of 2,048 references each), compared with the oracle."""
    from synth.configs import LLAMA32K
    cfg = LLAMA32K.with_(B=16, gather_frac=None)
    _log(f"[case] append bench shape B=16 T=32k proj={proj}")
    c = _make(cfg, prefill=True, proj=proj)
    pos = np.array([cfg.T - 1 - 3 * b for b in range(cfg.B)])
    c.append(pos)
    c.check("bench shape")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@PROJ
def test_append_exact_ties_keep_smaller_positions(dtype, proj):
    """The encode's exact-tie case on the append path: six references are
    one identical row, a later reference equals the appended tokens, so each
    token keeps that reference and the three smallest duplicate positions
    ([RKV] §2.1, the (d, j) order), with no tie excused."""
    from synth.configs import LLAMA8K
    from oracle import rkv_oracle as O
    cfg = LLAMA8K.with_(name=f"append_ties_{dtype}", B=1, T=1024, N=2, D=32, d_ff=64, d_c=64,
                        k=4, g=32, b=4, stride=8, n_protos=8, dtype=dtype)
    w = generate(cfg)
    kv = w.kv_f32()[0].astype(np.float32)
    s = cfg.stride
    dup = [s * m for m in (3, 5, 9, 12, 20, 21)]
    close, probes = s * 30, [250, 301, 517, 1001]
    rng = np.random.default_rng(5)
    base = kv[dup[0]].copy()
    probe = base + 0.1 * np.abs(base).mean() * rng.standard_normal(cfg.C).astype(np.float32)
    for t in dup:
        kv[t] = base
    for t in [close] + probes:
        kv[t] = probe
    if dtype == "bf16":
        u = kv.view(np.uint32)
        w.kv[0] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    else:
        w.kv[0] = kv
    _log(f"[case] append exact ties {dtype}")
    c = Cache(w, prefill_refs=True, proj=proj)
    for t in probes:
        c.append(np.array([t]))
    torch.cuda.synchronize()
    got = c.ref_idx.cpu().numpy()[0]
    want = np.sort(np.array([close] + dup[:3]))
    for t in probes:
        assert np.array_equal(got[t], want), (t, got[t], want)
    c.check(cfg.name)



_KNOB_BITS = {}      # records of the four-slice runs, one per distance batch size


@pytest.mark.parametrize("split,batch,rb", [(1, 2, 2), (2, 4, 2), (2, 2, 4), (4, 2, 4), (4, 4, 4)])
def test_append_row_slices_and_distance_batches(monkeypatch, split, batch, rb):
    """Every slicing of the C rows in the projection (the slices' partial
    sums are added in slice order, so each slicing has its own fp32 sums),
    two or four tokens per projection workgroup, and both distance batch
    sizes (the same bits) match the oracle; five sequences leave the last
    block of two or four tokens part empty."""
    cfg = LLAMA8K.with_(name=f"append_split{split}_u{batch}_rb{rb}", B=5, T=4096)
    monkeypatch.setenv("RKV_APP_SPLIT", str(split))
    monkeypatch.setenv("RKV_APP_DIST_U", str(batch))
    monkeypatch.setenv("RKV_APP_RB", str(rb))
    _log(f"[case] append {cfg.name}")
    c = _make(cfg, prefill=True)
    rng = np.random.default_rng(split)              # the same positions for both batch sizes
    for i in range(3):
        pos = rng.integers(1, cfg.T, size=cfg.B)
        if i == 1:
            pos[2] = -1
        c.append(pos)
    c.check(cfg.name)
    if split == 4:
        torch.cuda.synchronize()
        got = [t.cpu().numpy().view(np.uint8) for t in (c.codes, c.scale, c.zmin, c.ref_idx)]
        _KNOB_BITS[batch] = got
        if len(_KNOB_BITS) == 2:
            for a, b in zip(_KNOB_BITS[2], _KNOB_BITS[4]):
                assert np.array_equal(a, b), "the distance batch sizes gave different records"


@pytest.mark.parametrize("B", [1, 3])
@PROJ
def test_append_with_no_position_is_a_no_op(B, proj):
    """A call in which no sequence appends (every position -1 or T) writes
    nothing: records keep their pattern, the cache its rows."""
    cfg = RAGGED_BF16.with_(name=f"append_none_b{B}", B=B)
    _log(f"[case] append {cfg.name} no positions")
    c = _make(cfg, prefill=True, proj=proj)
    ref_proj = c.ref_proj.cpu().numpy().copy() if proj else None
    for pos in (np.full(B, -1), np.full(B, cfg.T), np.array([-1, cfg.T, -5][:B])):
        c.append(pos)
    torch.cuda.synchronize()
    assert not c.appended.any()
    assert (c.codes.cpu().numpy() == SENTINEL).all()
    assert (c.ref_idx.cpu().numpy().view(np.uint8) == SENTINEL).all()
    assert (c.scale.cpu().numpy().view(np.uint8) == SENTINEL).all()
    assert (c.z.cpu().numpy().view(np.uint8) == SENTINEL).all()
    kv = c.kv.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kv, c.expected_kv.view(np.uint16))
    if proj:
        assert np.array_equal(c.ref_proj.cpu().numpy().view(np.uint32), ref_proj.view(np.uint32))


@pytest.mark.parametrize("cfg", [RAGGED_BF16, RAGGED_F32,
                                 RAGGED_BF16.with_(name="append_ragged_bf16_fp8ref", ref_fp8=True),
                                 WIDE_FF, LLAMA8K.with_(B=2)],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("valu", [False, True], ids=["default", "valu"])
def test_project_refs_against_fp64(cfg, valu, monkeypatch):
    """rkv_project_refs: every stored reference's r_j [W1 | W2] against the
    fp64 product of the stored values (E4M3 values for an FP8 store); fp32
    sums over C rows of exact products, so within 1e-5 of the row's scale.
    bf16 input-precision references take the matrix cores unless
    RKV_REF_PROJ_VALU is set."""
    from oracle import rkv_oracle as O
    if valu:
        monkeypatch.setenv("RKV_REF_PROJ_VALU", "1")
    w = generate(cfg)
    _log(f"[case] project refs {cfg.name} valu={valu}")
    c = Cache(w, prefill_refs=True, proj=True)
    torch.cuda.synchronize()
    refs = np.asarray(R.rkv_reference_positions(c.p))
    W = np.concatenate([x.astype(np.float64) for x in w.weights_f32()[:2]], axis=1)
    got = c.ref_proj.cpu().numpy().reshape(cfg.B, len(refs), 2 * cfg.d_ff)
    kv = w.kv_f32().astype(np.float64)
    for b in range(cfg.B):
        rows = kv[b, refs]
        if cfg.ref_fp8:
            rows = O.fp8_e4m3(rows)
        want = rows @ W
        scale = np.abs(rows) @ np.abs(W)
        err = np.abs(got[b] - want) / np.maximum(scale, 1e-30)
        assert err.max() < 1e-5, (b, err.max())


def test_append_proj_extends_the_projections():
    """Filling an empty cache through rkv_append_proj writes each appended
    reference's row of the projections: they match rkv_project_refs of the
    filled cache within fp32 summation order."""
    cfg = RAGGED_BF16.with_(name="append_proj_rows", B=2, T=300)
    w = generate(cfg)
    _log("[case] append_proj projection rows")
    c = Cache(w, prefill_refs=False, proj=True)
    for t in range(cfg.T):
        c.append(np.full(cfg.B, t))
    torch.cuda.synchronize()
    built = c.ref_proj.cpu().numpy().copy()
    c.project()
    torch.cuda.synchronize()
    fresh = c.ref_proj.cpu().numpy()
    assert np.all(np.isfinite(built))
    assert np.allclose(built, fresh, rtol=1e-5, atol=1e-5 * np.abs(fresh).max())
