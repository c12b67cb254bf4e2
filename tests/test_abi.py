"""CPU tests of the C ABI: the library loads without a GPU, exports every
symbol include/rkv.h declares, and rejects bad arguments on the host before
anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import reference_residual_encoding_amd as R
from synth.configs import CONFIGS, LLAMA32K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # aligned, never dereferenced: validation fails first
FAKE_MIS = 0x10004      # misaligned


def header_functions():
    text = open(os.path.join(ROOT, "include", "rkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = R.lib()
    declared = header_functions()
    assert set(declared) == set(R.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert R.rkv_abi_version() == R.RKV_ABI_VERSION


def test_status_strings():
    assert R.rkv_status_str(0) == "RKV_OK"
    assert R.rkv_status_str(3) == "RKV_ERR_WORKSPACE"


def _p(cfg, **kw):
    d = dict(B=cfg.B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k, g=cfg.g,
             b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
             ref_alpha=cfg.alpha, ref_format="fp8" if cfg.ref_fp8 else "input")
    d.update(kw)
    return R.params(**d)


def _encode(p, ws_bytes=1 << 40, **ptrs):
    args = dict(kv=FAKE, w1=FAKE, w2=FAKE, w3=FAKE, ref_idx=FAKE, codes=FAKE, scale=FAKE,
                zmin=FAKE, z=None, workspace=FAKE)
    args.update(ptrs)
    # Safety: these pointers are fake; a call that would pass validation must
    # never be made (it would enqueue kernels on them).
    valid_ptrs = all(v is not None and v % 16 == 0 for k, v in args.items() if k != "z") \
        and (args["z"] is None or args["z"] % 16 == 0)
    if R.rkv_encode_workspace_bytes(p) and valid_ptrs and ws_bytes >= R.rkv_encode_workspace_bytes(p):
        pytest.fail("test would pass validation with fake pointers")
    return R.rkv_encode(p, args["kv"], args["w1"], args["w2"], args["w3"], args["ref_idx"],
                        args["codes"], args["scale"], args["zmin"], args["z"],
                        args["workspace"], ws_bytes, None, check=False)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_workspace_size_is_positive_and_grows_with_T(cfg):
    w = R.rkv_encode_workspace_bytes(_p(cfg))
    assert w > 0 and w % 256 == 0
    assert R.rkv_encode_workspace_bytes(_p(cfg, T=cfg.T * 2)) > w


def test_workspace_size_zero_for_invalid_params():
    assert R.rkv_encode_workspace_bytes(_p(LLAMA32K, b=3)) == 0


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, R.RKV_ERR_INVALID_ARG), ("T", -1, R.RKV_ERR_INVALID_ARG),
    ("N", 0, R.RKV_ERR_INVALID_ARG), ("d_ff", 0, R.RKV_ERR_INVALID_ARG),
    ("k", 0, R.RKV_ERR_INVALID_ARG), ("ref_stride", 0, R.RKV_ERR_INVALID_ARG),
    ("b", 3, R.RKV_ERR_INVALID_ARG), ("b", 8, R.RKV_ERR_INVALID_ARG),
    ("g", 0, R.RKV_ERR_INVALID_ARG), ("dtype", 7, R.RKV_ERR_INVALID_ARG),
    ("g", 24, R.RKV_ERR_UNSUPPORTED), ("k", 9, R.RKV_ERR_UNSUPPORTED),
    ("d_c", 48, R.RKV_ERR_UNSUPPORTED), ("g", 64, R.RKV_ERR_UNSUPPORTED),
    ("d_ff", 1000, R.RKV_ERR_UNSUPPORTED), ("D", 10, R.RKV_ERR_UNSUPPORTED),
    ("d_c", 65536 + 32, R.RKV_ERR_UNSUPPORTED), ("d_ff", 65536 + 32, R.RKV_ERR_UNSUPPORTED),
    ("ref_alpha", -0.5, R.RKV_ERR_INVALID_ARG), ("ref_alpha", float("nan"), R.RKV_ERR_INVALID_ARG),
    ("n_sink", -1, R.RKV_ERR_INVALID_ARG),
])
def test_encode_rejects_bad_params(field, value, status):
    kw = {field: value}
    if field == "g" and value == 64:
        kw["d_c"] = 96         # 64 does not divide 96
    st = _encode(_p(LLAMA32K, **kw))
    assert st == status, R.rkv_last_error()
    assert R.rkv_last_error() != ""


@pytest.mark.parametrize("name", ["kv", "w1", "w2", "w3", "ref_idx", "codes", "scale", "zmin",
                                  "workspace"])
def test_encode_rejects_null_and_misaligned(name):
    p = _p(LLAMA32K)
    assert _encode(p, **{name: None}) == R.RKV_ERR_INVALID_ARG
    assert name in R.rkv_last_error()
    assert _encode(p, **{name: FAKE_MIS}) == R.RKV_ERR_INVALID_ARG
    assert "aligned" in R.rkv_last_error()
    assert _encode(p, z=FAKE_MIS) == R.RKV_ERR_INVALID_ARG


def test_encode_rejects_small_workspace():
    p = _p(LLAMA32K)
    need = R.rkv_encode_workspace_bytes(p)
    assert _encode(p, ws_bytes=need - 1) == R.RKV_ERR_WORKSPACE
    assert str(need) in R.rkv_last_error()
    st = R.rkv_select(p, FAKE, FAKE, FAKE, need - 256, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE


def test_raising_wrapper_carries_status_and_text():
    with pytest.raises(R.RkvError) as e:
        R.rkv_encode(_p(LLAMA32K, b=5), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                     FAKE, 1 << 40, None)
    assert e.value.status == R.RKV_ERR_INVALID_ARG and "b must be" in str(e.value)


def test_gather_and_quantize_validation_and_empty_calls():
    p = _p(LLAMA32K)
    # zero-size calls succeed without touching the device
    assert R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, FAKE, 0, FAKE, "f32", None, check=False) == 0
    assert R.rkv_quantize(p, FAKE, 0, FAKE, FAKE, FAKE, None, check=False) == 0
    assert R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, FAKE, -1, FAKE, "f32", None,
                                check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, None, 5, FAKE, "f32", None,
                                check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, FAKE, 5, FAKE, 9, None,
                                check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_dequant_gather(_p(LLAMA32K, b=1), FAKE, FAKE, FAKE, FAKE, 5, FAKE, "f32", None,
                                check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_quantize(p, FAKE, -3, FAKE, FAKE, FAKE, None, check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_quantize(p, FAKE_MIS, 3, FAKE, FAKE, FAKE, None, check=False) == R.RKV_ERR_INVALID_ARG


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "reference_residual_encoding_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "rkv_oracle" not in text, f


def _restore(p, n_idx=4, ws_bytes=1 << 40, theta=10000.0, out_dtype=R.RKV_F32, **ptrs):
    args = dict(codes=FAKE, scale=FAKE, zmin=FAKE, ref_idx=FAKE, kv=FAKE, wd=FAKE, idx=FAKE,
                out=FAKE, workspace=FAKE)
    args.update(ptrs)
    need = R.rkv_restore_workspace_bytes(p, max(n_idx, 0))
    valid_ptrs = all(v is not None and v % 16 == 0 for v in args.values())
    if need and n_idx > 0 and valid_ptrs and ws_bytes >= need and theta == theta \
            and out_dtype in (R.RKV_F32, R.RKV_BF16):
        pytest.fail("test would pass validation with fake pointers")
    return R.rkv_restore(p, args["codes"], args["scale"], args["zmin"], args["ref_idx"], args["kv"],
                         args["wd"], args["idx"], n_idx, theta, args["out"], out_dtype,
                         args["workspace"], ws_bytes, None, check=False)


def test_restore_validation():
    p = _p(LLAMA32K)
    assert R.rkv_restore_workspace_bytes(p, 9830) > R.rkv_restore_workspace_bytes(p, 10) > 0
    assert R.rkv_restore_workspace_bytes(_p(LLAMA32K, D=96, N=8), 10) == 0   # D must divide 128
    assert _restore(_p(LLAMA32K, D=96), codes=None) == R.RKV_ERR_UNSUPPORTED
    assert _restore(p, n_idx=-1) == R.RKV_ERR_INVALID_ARG
    assert _restore(p, out=None) == R.RKV_ERR_INVALID_ARG
    assert _restore(p, wd=FAKE_MIS) == R.RKV_ERR_INVALID_ARG
    assert _restore(p, ws_bytes=1024) == R.RKV_ERR_WORKSPACE
    assert _restore(p, theta=float("nan")) == R.RKV_ERR_INVALID_ARG
    assert _restore(p, out_dtype=5) == R.RKV_ERR_INVALID_ARG
    # n_idx == 0 is a no-op and touches no pointer
    assert R.rkv_restore(p, None, None, None, None, None, None, None, 0, 1.0, None, R.RKV_F32,
                         None, 0, None, check=False) == R.RKV_OK


def test_dynamic_schedule_shrinks_the_workspace():
    """Fewer references under a growing schedule ([RKV] §2.6) need fewer
    reference rows and projections."""
    from synth.configs import LLAMA32K_DYN
    assert 0 < R.rkv_encode_workspace_bytes(_p(LLAMA32K_DYN)) < R.rkv_encode_workspace_bytes(_p(LLAMA32K))


def _append(p, ws_bytes=1 << 40, **ptrs):
    args = dict(kv=FAKE, kv_new=FAKE, pos=FAKE, w1=FAKE, w2=FAKE, w3=FAKE, ref_idx=FAKE,
                codes=FAKE, scale=FAKE, zmin=FAKE, z=None, workspace=FAKE)
    args.update(ptrs)
    valid_ptrs = all(v is not None and v % 16 == 0 for k, v in args.items() if k != "z") \
        and (args["z"] is None or args["z"] % 16 == 0)
    need = R.rkv_append_workspace_bytes(p)
    if need and valid_ptrs and ws_bytes >= need:
        pytest.fail("test would pass validation with fake pointers")
    return R.rkv_append(p, args["kv"], args["kv_new"], args["pos"], args["w1"], args["w2"],
                        args["w3"], args["ref_idx"], args["codes"], args["scale"], args["zmin"],
                        args["z"], args["workspace"], ws_bytes, None, check=False)


@pytest.mark.parametrize("name", ["kv", "kv_new", "pos", "w1", "w2", "w3", "ref_idx", "codes",
                                  "scale", "zmin", "workspace"])
def test_append_rejects_null_and_misaligned(name):
    p = _p(LLAMA32K)
    assert _append(p, **{name: None}) == R.RKV_ERR_INVALID_ARG
    assert _append(p, **{name: FAKE_MIS}) == R.RKV_ERR_INVALID_ARG


def test_append_validation_and_workspace():
    p = _p(LLAMA32K)
    need = R.rkv_append_workspace_bytes(p)
    # a few vectors per sequence and one partial list per 8 pool references
    assert 0 < need < 1 << 20
    assert R.rkv_append_workspace_bytes(_p(LLAMA32K, B=16)) > need
    assert _append(p, ws_bytes=need - 1) == R.RKV_ERR_WORKSPACE
    assert _append(_p(LLAMA32K, k=9)) == R.RKV_ERR_UNSUPPORTED
    assert _append(_p(LLAMA32K, ref_alpha=-1.0)) == R.RKV_ERR_INVALID_ARG
    assert _append(p, z=FAKE_MIS) == R.RKV_ERR_INVALID_ARG


def test_reference_positions_host_query():
    """The schedule of [RKV] §2.6 as host data, with no device work."""
    assert R.rkv_reference_positions(_p(LLAMA32K, T=100)) == list(range(0, 100, 16))
    got = R.rkv_reference_positions(_p(LLAMA32K, T=80, ref_stride=10, ref_alpha=0.1, n_sink=3))
    # sinks 0..2, then p0 = 3, gaps 10 + floor(0.1 (p - 3))
    assert got == [0, 1, 2, 3, 13, 24, 36, 49, 63, 79]
    with pytest.raises(R.RkvError):
        R.rkv_reference_positions(_p(LLAMA32K, ref_stride=0))


def test_identity_mode_validation():
    """b = 16 is the identity mode ([RKV] §2.4): larger records, no group numbers."""
    p16 = _p(LLAMA32K, b=16)
    assert R.rkv_encode_workspace_bytes(p16) > 0
    assert R.rkv_encode_workspace_bytes(_p(LLAMA32K, b=8)) == 0
    assert R.rkv_encode_workspace_bytes(_p(LLAMA32K, b=16, g=0)) > 0       # g is not read
    assert _encode(_p(LLAMA32K, b=3)) == R.RKV_ERR_INVALID_ARG
    # scale / zmin may be NULL in identity mode: validation then stops at the next pointer
    assert _encode(p16, scale=None, zmin=None, workspace=None) == R.RKV_ERR_INVALID_ARG
    assert "workspace" in R.rkv_last_error()


def test_fp8_reference_format_validation():
    """ref_format selects how the cache keeps its references ([RKV] §2.4)."""
    assert R.rkv_encode_workspace_bytes(_p(LLAMA32K, ref_format="fp8")) > 0
    assert _encode(_p(LLAMA32K, ref_format=7)) == R.RKV_ERR_INVALID_ARG
    st = R.rkv_store_refs(_p(LLAMA32K), FAKE, FAKE, None, check=False)
    assert st == R.RKV_ERR_INVALID_ARG and "RKV_REF_FP8" in R.rkv_last_error()
    assert R.rkv_store_refs(_p(LLAMA32K, ref_format="fp8"), FAKE, None, None,
                            check=False) == R.RKV_ERR_INVALID_ARG
    assert R.rkv_store_refs(_p(LLAMA32K, ref_format="fp8"), FAKE_MIS, FAKE, None,
                            check=False) == R.RKV_ERR_INVALID_ARG


class _FakeGpuTensor:
    """Stands in for a GPU tensor on this CPU-only host: the binding reads only
    is_cuda, is_contiguous(), dtype, numel(), element_size() before a call, and
    every case below fails those checks, so data_ptr() is never reached."""

    def __init__(self, dtype="torch.bfloat16", numel=1 << 40, esize=2, contiguous=True):
        self.is_cuda, self.dtype, self._n, self._e, self._c = True, dtype, numel, esize, contiguous
        self.device = "cuda:0"

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def data_ptr(self):
        raise AssertionError("validation should have failed before data_ptr()")


def test_binding_rejects_host_strided_mistyped_and_short_tensors():
    """The binding checks every tensor before the library is called: a CPU
    tensor, a non-contiguous view, the wrong dtype for kv / weights, or a
    buffer shorter than the call's layout raise ValueError, so no such
    pointer can reach a kernel."""
    import torch
    p = _p(LLAMA32K)
    good = _FakeGpuTensor()
    cases = {
        "host": torch.zeros(4, dtype=torch.bfloat16),
        "strided": _FakeGpuTensor(contiguous=False),
        "dtype": _FakeGpuTensor(dtype="torch.float32", esize=4),
        "short": _FakeGpuTensor(numel=100),
    }
    for what, bad in cases.items():
        with pytest.raises(ValueError):
            R.rkv_encode(p, bad, good, good, good, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
        with pytest.raises(ValueError):
            R.rkv_encode(p, FAKE, FAKE, FAKE, bad, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
        with pytest.raises(ValueError):
            R.rkv_select(p, bad, FAKE, FAKE, 1 << 40, None)
        with pytest.raises(ValueError):
            R.rkv_restore(p, FAKE, FAKE, FAKE, FAKE, bad, FAKE, FAKE, 10, 1.0, FAKE, "f32", FAKE,
                          1 << 40, None)
        with pytest.raises(ValueError):
            R.rkv_append(p, FAKE, bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                         1 << 40, None)
        with pytest.raises(ValueError):
            R.rkv_store_refs(_p(LLAMA32K, ref_format="fp8"), bad, FAKE, None)
    # index and output buffers: dtype and size follow n_idx and out_dtype
    with pytest.raises(ValueError):
        R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, _FakeGpuTensor("torch.int64", esize=8), 5, FAKE,
                             "f32", None)
    with pytest.raises(ValueError):
        R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, FAKE, 1000, _FakeGpuTensor("torch.float32", 1000, 4),
                             "f32", None)
    with pytest.raises(ValueError):
        R.rkv_dequant_gather(p, FAKE, FAKE, FAKE, FAKE, 5, _FakeGpuTensor("torch.float32", esize=4),
                             "bf16", None)


def test_noalloc_append_rejects_calls_beyond_its_fixed_scratch():
    """rkv_append_noalloc works in a fixed 4 MiB device array: a call that
    needs more is refused on the host (RKV_ERR_WORKSPACE) before any device
    call, with a message naming the alternative."""
    from synth.configs import LLAMA8K
    p = _p(LLAMA8K, B=900, T=4096)
    assert R.rkv_append_workspace_bytes(p) > 4 << 20      # so validation cannot pass
    st = R.rkv_append_noalloc(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                              None, check=False)
    assert st == R.RKV_ERR_WORKSPACE
    assert "rkv_append with a workspace" in R.rkv_last_error()
    assert R.rkv_append_noalloc(p, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None, None, check=False) == R.RKV_ERR_INVALID_ARG


def test_packed_weights_calls_check_sizes_on_the_host():
    """rkv_pack_weights / rkv_encode_packed refuse a packed buffer (or a
    workspace) smaller than their layout before anything is enqueued."""
    p = _p(LLAMA32K)
    need = R.rkv_packed_weights_bytes(p)
    # W1|W2 interleaved (2 d_ff x C) plus W3 as K-contiguous rows (d_c x d_ff), bf16
    assert need == 2 * 1024 * 2048 * 2 + 512 * 1024 * 2
    assert R.rkv_packed_weights_bytes(_p(LLAMA32K, b=5)) == 0
    st = R.rkv_pack_weights(p, FAKE, FAKE, FAKE, FAKE, need - 1, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE and str(need) in R.rkv_last_error()
    st = R.rkv_encode_packed(p, FAKE, FAKE, need - 256, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                             1 << 40, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE
    ws = R.rkv_encode_workspace_bytes(p)
    st = R.rkv_encode_packed(p, FAKE, FAKE, need, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 256,
                             None, check=False)
    assert st == R.RKV_ERR_WORKSPACE
    assert R.rkv_encode_packed(p, FAKE, None, need, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None,
                               check=False) == R.RKV_ERR_INVALID_ARG


def test_packed_decoder_calls_check_sizes_on_the_host():
    """rkv_pack_decoder / rkv_restore_packed refuse a packed decoder buffer
    (or a workspace) smaller than their layout, and a NULL packed buffer,
    before anything is enqueued."""
    p = _p(LLAMA32K)
    need = R.rkv_packed_decoder_bytes(p)
    # W_d as C rows of the d_c latents, bf16
    assert need == 2048 * 512 * 2
    assert R.rkv_packed_decoder_bytes(_p(LLAMA32K, D=96)) == 0      # restore needs D | 128
    st = R.rkv_pack_decoder(p, FAKE, FAKE, need - 1, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE and str(need) in R.rkv_last_error()
    n = 100
    ws = R.rkv_restore_workspace_bytes(p, n)
    st = R.rkv_restore_packed(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, FAKE, n, 1e4,
                              FAKE, "bf16", FAKE, ws, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE
    st = R.rkv_restore_packed(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, FAKE, n, 1e4, FAKE,
                              "bf16", FAKE, ws - 256, None, check=False)
    assert st == R.RKV_ERR_WORKSPACE
    st = R.rkv_restore_packed(p, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, FAKE, n, 1e4, FAKE,
                              "bf16", FAKE, ws, None, check=False)
    assert st == R.RKV_ERR_INVALID_ARG and "packed" in R.rkv_last_error()
    assert R.rkv_restore_packed(p, None, None, None, None, None, None, 0, None, 0, 1e4, None,
                                "bf16", None, 0, None) == R.RKV_OK             # nothing to do


def test_encode_workspace_size_does_not_depend_on_the_tiling(monkeypatch):
    """The distance launch's tiling (wide, narrow, or narrow on 128-reference
    chunks) is chosen per shape, or forced by RKV_DIST_TILE; the list buffer
    is sized for the smallest chunk, so a workspace sized once fits every
    tiling."""
    from synth.configs import LLAMA8K
    for cfg in (LLAMA32K, LLAMA8K):
        p = _p(cfg)
        sizes = set()
        for tiling in ("wide", "narrow", "short", None):
            if tiling is None:
                monkeypatch.delenv("RKV_DIST_TILE", raising=False)
            else:
                monkeypatch.setenv("RKV_DIST_TILE", tiling)
            sizes.add(R.rkv_encode_workspace_bytes(p))
        assert len(sizes) == 1 and sizes.pop() > 0
