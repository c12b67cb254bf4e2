"""Guard bands: every output buffer of the encode, the gather and the
restore sits between two 4 KiB canary regions filled with a byte pattern;
after the call both regions must be untouched, so a write before or past
the end of ref_idx, codes, scale, zmin, z, the workspace or out would show.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import reference_residual_encoding_amd as R
from synth import decoder_weight, generate
from synth.configs import LLAMA32K, LLAMA8K, MM_INT2, TINY

import rkv_parity as P

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """A device buffer with canaries before and after its payload."""

    def __init__(self, shape, dtype):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = nbytes
        self.raw = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + nbytes].view(dtype).view(*shape) if nbytes else \
            torch.empty(shape, dtype=dtype, device="cuda")

    def intact(self):
        h = self.raw.cpu().numpy()
        return bool((h[:GUARD] == PATTERN).all() and (h[GUARD + self.n:] == PATTERN).all())


def _log(msg):
    print(msg, flush=True)


RAGGED = LLAMA8K.with_(name="guard_ragged_bf16_b2", B=3, T=1000, N=2, D=32, d_ff=96, d_c=64,
                       k=5, g=16, b=2, stride=7, n_protos=24)


@pytest.mark.parametrize("cfg", [TINY, RAGGED, TINY.with_(name="guard_identity", b=16),
                                 LLAMA32K, MM_INT2], ids=lambda c: c.name)
def test_encode_gather_restore_stay_inside_their_buffers(cfg):
    _log(f"[case] guard {cfg.name}")
    w = generate(cfg)
    p = P.params_of(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, T = cfg.B, cfg.T
    ng = 0 if cfg.b == 16 else cfg.d_c // cfg.g
    kv = P.to_device(w.kv, cfg.dtype)
    w1, w2, w3 = (P.to_device(x, cfg.dtype) for x in (w.w1, w.w2, w.w3))
    g = dict(ref_idx=Guarded((B, T, cfg.k), torch.int32),
             codes=Guarded((B, T, cfg.d_c * cfg.b // 8), torch.uint8),
             scale=Guarded((B, T, ng), torch.float16), zmin=Guarded((B, T, ng), torch.float16),
             z=Guarded((B, T, cfg.d_c), torch.float32))
    ws_bytes = R.rkv_encode_workspace_bytes(p)
    g["workspace"] = Guarded((ws_bytes,), torch.uint8)
    st = torch.cuda.current_stream()
    R.rkv_encode(p, kv, w1, w2, w3, g["ref_idx"].t, g["codes"].t, g["scale"].t if ng else None,
                 g["zmin"].t if ng else None, g["z"].t, g["workspace"].t, ws_bytes, st)
    # gather: the workload's subset (or every position) plus out-of-range rows
    idx = np.asarray(w.gather_idx, np.int32) if cfg.gather_frac else np.arange(B * T, dtype=np.int32)
    idx = np.concatenate([idx, [-1, B * T]]).astype(np.int32)
    d_idx = torch.from_numpy(idx).cuda()
    n = len(idx)
    g["gather_f32"] = Guarded((n, cfg.d_c), torch.float32)
    g["gather_bf16"] = Guarded((n, cfg.d_c), torch.bfloat16)
    for key, od in (("gather_f32", "f32"), ("gather_bf16", "bf16")):
        R.rkv_dequant_gather(p, g["codes"].t, g["scale"].t if ng else None,
                             g["zmin"].t if ng else None, d_idx, n, g[key].t, od, st)
    # restore of the same rows
    wd = P.to_device(decoder_weight(cfg), cfg.dtype)
    rws = R.rkv_restore_workspace_bytes(p, n)
    g["restore_ws"] = Guarded((rws,), torch.uint8)
    g["restore_out"] = Guarded((n, cfg.C), dt)
    R.rkv_restore(p, g["codes"].t, g["scale"].t if ng else None, g["zmin"].t if ng else None,
                  g["ref_idx"].t, kv, wd, d_idx, n, cfg.rope_theta, g["restore_out"].t,
                  cfg.dtype, g["restore_ws"].t, rws, st)
    torch.cuda.synchronize()
    bad = [k for k, v in g.items() if not v.intact()]
    assert not bad, f"{cfg.name}: canary overwritten around {bad}"
    # the payloads were written (a quick sanity check, not parity)
    assert int((g["ref_idx"].t >= 0).sum()) > 0 or T <= cfg.stride
    assert torch.isnan(g["gather_f32"].t[-2:]).all() and not torch.isnan(g["gather_f32"].t[:-2]).any()
