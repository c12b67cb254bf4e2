"""CPU tests of the host logic around the GPU path: the library's host-side
schedule against the oracle's, the benchmark's algorithmic work counts, and
the one-GPU guard of bench.py.  No GPU and no device call."""
import os
import subprocess
import sys

import numpy as np
import pytest

import reference_residual_encoding_amd as R
from oracle import rkv_oracle as O
from synth.configs import CONFIGS, DYNAMIC, LLAMA32K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _params(cfg, **kw):
    d = dict(B=cfg.B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k, g=cfg.g,
             b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
             ref_alpha=cfg.alpha)
    d.update(kw)
    return R.params(**d)


@pytest.mark.parametrize("cfg", list(CONFIGS) + list(DYNAMIC), ids=lambda c: c.name)
def test_library_schedule_equals_the_oracle_schedule(cfg):
    """The C++ host schedule (rkv_reference_positions) and the oracle's
    Python recurrence ([RKV] §2.6) are separate implementations."""
    got = R.rkv_reference_positions(_params(cfg))
    want = O.reference_schedule(cfg.T, cfg.stride, cfg.alpha, cfg.n_sink)
    assert got == want.tolist()


@pytest.mark.parametrize("T,s0,alpha,n_sink", [(1, 1, 0.0, 0), (7, 3, 0.0, 9), (5000, 4, 0.3, 2),
                                               (262144, 10, 0.001, 0), (100, 1, 2.0, 0)])
def test_library_schedule_special_cases(T, s0, alpha, n_sink):
    p = _params(LLAMA32K, T=T, ref_stride=s0, ref_alpha=alpha, n_sink=n_sink)
    assert R.rkv_reference_positions(p) == O.reference_schedule(T, s0, alpha, n_sink).tolist()


def test_benchmark_work_counts():
    """Algorithmic work of the long-context workload: the causal pair count
    (every non-reference token against the references before it), the
    distance launch's flops (those pairs, plus the reference projection that
    runs in the same launch) and the token projection's flops, from the
    schedule by brute force."""
    cfg = LLAMA32K
    refs = O.reference_schedule(cfg.T, cfg.stride)
    nref, nr, pairs = bench.schedule_counts(refs, cfg.T)
    assert (nref, nr) == (2048, 30720)
    assert pairs == sum(-(-t // cfg.stride) for t in range(cfg.T) if t % cfg.stride)
    work = bench.stage_work(cfg, 9830, refs)
    assert work["dist"] == ("flops", 2.0 * cfg.C * pairs + 2.0 * cfg.C * 2 * cfg.d_ff * nref)
    assert "proj" not in work
    assert work["swiglu"] == ("flops", 2.0 * cfg.C * 2 * cfg.d_ff * nr)
    assert work["swiglu"][1] == 257698037760.0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
