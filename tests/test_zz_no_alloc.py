"""The allocation-free append (rkv_append_noalloc, for callers that cannot
allocate device memory) against rkv_append with a caller workspace: the same
records, latents and cache rows, bit for bit, on two calls in a row (the
second with fewer sequences, a growing schedule, and the scratch still
holding the first call's contents), each also checked against the oracle.
Needs an MI355X."""
import numpy as np
import pytest
import torch

import reference_residual_encoding_amd as R
from synth import generate
from synth.configs import LLAMA8K, LLAMA8K_DYN

import rkv_parity as P
from test_gpu_append import Cache

pytestmark = pytest.mark.gpu


class NoAllocCache(Cache):
    """The same cache, appended through rkv_append_noalloc."""

    def append(self, pos):
        cfg = self.cfg
        pos = np.asarray(pos, dtype=np.int64)
        rows = np.zeros((cfg.B, cfg.C), dtype=self.w.kv.dtype)
        for b, t in enumerate(pos):
            if 0 <= t < cfg.T:
                rows[b] = self.w.kv[b, t]
                self.appended[b, t] = True
                if self.ref_mask[t]:
                    self.expected_kv[b, t] = self.w.kv[b, t]
        kv_new = P.to_device(rows, cfg.dtype)
        d_pos = torch.from_numpy(pos.astype(np.int32)).cuda()
        R.rkv_append_noalloc(self.p, self.kv, kv_new, d_pos, self.w1, self.w2, self.w3,
                             self.ref_idx, self.codes, self.scale, self.zmin, self.z,
                             torch.cuda.current_stream())


def _same(a, b, name):
    torch.cuda.synchronize()
    for key in ("ref_idx", "codes", "scale", "zmin", "z", "kv"):
        x, y = getattr(a, key).cpu(), getattr(b, key).cpu()
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{name}: {key} differs"


def test_noalloc_append_matches_workspace_append_on_two_calls():
    calls = [
        # 8 sequences at the end of an 8k context (pools of 512 references),
        # one reference position among them
        (LLAMA8K.with_(name="noalloc_llama_B8", B=8),
         lambda cfg: np.array([cfg.T - 1 - 5 * b for b in range(cfg.B - 1)] + [cfg.T - 16])),
        # then a smaller call: 2 sequences, growing schedule, one skipped slot
        (LLAMA8K_DYN.with_(name="noalloc_llama_dyn_B2", B=2),
         lambda cfg: np.array([cfg.T // 2 + 7, -1])),
    ]
    for cfg, positions in calls:
        print(f"[case] noalloc {cfg.name}", flush=True)
        w = generate(cfg)
        ref = Cache(w, prefill_refs=True)
        mine = NoAllocCache(w, prefill_refs=True)
        pos = positions(cfg)
        ref.append(pos)
        mine.append(pos)
        _same(ref, mine, cfg.name)
        mine.check(cfg.name)

