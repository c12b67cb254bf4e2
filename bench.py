#!/usr/bin/env python3
"""Benchmark of the ResidualKV cache-write path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the encode over B*T tokens (reference retrieval, reference mean, SwiGLU
compressor residual, group quantiser; rkv_encode_packed, the compressor's
weights packed once beforehand by rkv_pack_weights) followed by
rkv_dequant_gather of the workload's selected token subset.  Inputs are
resident in HBM before the timed region starts.  The line also gives the
step through rkv_encode, which repacks the weights at every call.  Prints
one JSON line.

Workload (default): Llama-3.1-8B single-layer shape, B=1, T=32768, N=8, D=128
(C = 2048), d_ff=1024, d_c=512, k=4, reference stride 16, INT4, g=32; gather
of 30 % of the positions.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# kernel behind each profiled stage
STAGE_KERNEL = {"pack": "k_pack_weights", "norms": "k_setup", "dist": "k_dist_topk",
                "merge": "k_topk_merge", "swiglu": "k_swiglu",
                "w3": "k_w3_quant", "quant": "k_quantize", "gather": "k_gather"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.txt")


def source_digest() -> str:
    """sha256 over the HIP/C++ sources of librkv (file names and contents)."""
    import hashlib
    d = os.path.join(ROOT, "reference_residual_encoding_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel`, from the committed hardware-counter
    summary of this workload, or None when there is none or the kernel
    sources have changed since the counters were taken."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    digest, table = None, {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "source_sha256":
                digest = parts[1]
            elif len(parts) == 4 and parts[0].startswith("k_"):
                table[parts[0]] = float(parts[3])
    if digest != source_digest():
        return None
    return table.get(kernel)


def schedule_counts(refs, T: int):
    """(references, non-references, causal (token, reference) pairs) of one
    sequence, from the schedule's reference positions."""
    import numpy as np
    mask = np.zeros(T, dtype=bool)
    mask[np.asarray(refs, dtype=np.int64)] = True
    before = np.cumsum(mask) - mask                  # references before each position
    return int(mask.sum()), int(T - mask.sum()), int(before[~mask].sum())


def stage_work(cfg, n_gather: int, refs):
    """Algorithmic work of one launch of each stage: (kind, amount).

    MFMA stages count 2 flops per multiply-add of the contraction the method
    needs (the bf16 hi/lo split of the W3 input is not counted); HBM-bound
    stages count the bytes they must move.  `refs` are the schedule's
    reference positions (rkv_reference_positions)."""
    B, T, C = cfg.B, cfg.T, cfg.C
    nref, nr, pairs = schedule_counts(refs, T)
    pairs *= B
    esz = 2 if cfg.dtype == "bf16" else 4
    rec = cfg.d_c * cfg.b // 8 + 4 * (cfg.d_c // cfg.g)
    return {
        "pack": ("bytes", 2 * (2 * C * cfg.d_ff + cfg.d_ff * cfg.d_c) * esz),
        # set-up: weight repacking, schedule tables, reference rows and norms
        "norms": ("bytes", 2 * (2 * C * cfg.d_ff + cfg.d_ff * cfg.d_c) * esz + 3 * 4 * T
                  + 2 * B * nref * C * esz),
        # the distance scan, plus the reference projection P = R[W1|W2] whose
        # tiles run at the end of the same launch
        "dist": ("flops", 2.0 * C * pairs + 2.0 * C * 2 * cfg.d_ff * B * nref),
        "merge": ("bytes", B * T * cfg.k * 4),
        "swiglu": ("flops", 2.0 * C * 2 * cfg.d_ff * B * nr),
        "w3": ("flops", 2.0 * cfg.d_ff * cfg.d_c * B * nr),
        "quant": ("bytes", B * nr * cfg.d_c * 4 + B * T * rec),
        "gather": ("bytes", n_gather * (rec + cfg.d_c * 2)),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _oracle_encode_time(w, n_tokens: int, seed: int = 0):
    """Wall time of the oracle encoding n_tokens random non-reference tokens
    of sequence 0 (each on its own: retrieval over its causal pool, mean, two
    f_c, quantiser); n_tokens <= 0 takes every non-reference token."""
    import numpy as np
    from oracle import rkv_oracle as O
    cfg = w.cfg
    rng = np.random.default_rng(seed)
    kv = w.kv_f32()[0].astype(np.float64)
    W1, W2, W3 = (x.astype(np.float64) for x in w.weights_f32())
    mask = np.zeros(cfg.T, dtype=bool)
    mask[O.reference_schedule(cfg.T, cfg.stride, cfg.alpha, cfg.n_sink)] = True
    nonref = np.flatnonzero(~mask)
    pos = nonref if n_tokens <= 0 else np.sort(rng.choice(nonref, size=n_tokens, replace=False))
    t0 = time.perf_counter()
    enc = O.encode_tokens(kv, W1, W2, W3, pos, k=cfg.k, g=cfg.g, b=cfg.b, s=cfg.stride,
                          alpha=cfg.alpha, n_sink=cfg.n_sink)
    return len(pos), time.perf_counter() - t0, enc


def cpu_baseline(w, n_tokens: int, seed: int = 0):
    """The CPU oracle, as it stands, on a bounded sample of the workload,
    with all of the host's BLAS threads; then the same oracle on one thread
    (the tiny workload in full, and a sample of the 8k Llama shape), and the
    oracle's dequantise-gather of the workload's selected rows."""
    import numpy as np
    from oracle import rkv_oracle as O
    from synth import generate
    from synth.configs import LLAMA8K, TINY
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits, threads = None, 1
    cfg = w.cfg
    n, dt, enc = _oracle_encode_time(w, n_tokens, seed)
    out = {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} random non-reference tokens of sequence 0 of {cfg.name}, "
                     f"each encoded on its own (retrieval over its causal pool, mean, two f_c, "
                     f"quantiser), numpy fp64; {dt:.2f} s",
           "cpu_model": cpu_model(), "host_threads_visible": len(os.sched_getaffinity(0))}
    # the oracle's gather of the workload's rows (records of random latents
    # of the workload's shape: the gather's cost does not depend on values)
    rows = cfg.B * cfg.T
    rng = np.random.default_rng(seed + 1)
    q, dh, mh = O.quantize(rng.standard_normal((rows, cfg.d_c)), cfg.g, cfg.b)
    codes = O.pack_codes(q, cfg.b)
    t0 = time.perf_counter()
    O.gather(codes, dh, mh, w.gather_idx, g=cfg.g, b=cfg.b, d_c=cfg.d_c)
    gdt = time.perf_counter() - t0
    out["gather"] = {"rows": int(len(w.gather_idx)), "seconds": round(gdt, 4),
                     "rows_per_s": round(len(w.gather_idx) / gdt, 1)}
    if threadpool_limits is not None:
        one = {}
        with threadpool_limits(limits=1):
            for c, k in ((TINY, 0), (LLAMA8K, 256)):
                n1, dt1, _ = _oracle_encode_time(generate(c), k, seed)
                one[c.name] = {"tokens": n1, "seconds": round(dt1, 3),
                               "tokens_per_s": round(n1 / dt1, 1)}
        out["one_thread"] = one
    return out


def bench_restore(R, cfg, w, p, kv, out, idx, stream, args):
    """rkv_restore_packed of the gathered rows (decoder product z~ W_d,
    reference mean, RoPE on K; bf16 out) with W_d packed once by
    rkv_pack_decoder, timed on its own after the encode steps; the records
    are those the timed encode wrote.  rkv_restore, which repacks W_d at
    every call, is timed the same way beside it."""
    import numpy as np
    import torch
    from synth import decoder_weight
    dev = kv.device
    wd = decoder_weight(cfg)
    if cfg.dtype == "bf16":
        d_wd = torch.from_numpy(np.ascontiguousarray(wd).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        d_wd = torch.from_numpy(wd).to(dev)
    n = idx.numel()
    rout = torch.empty((n, cfg.C), dtype=torch.bfloat16, device=dev)
    wsb = R.rkv_restore_workspace_bytes(p, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    pkb = R.rkv_packed_decoder_bytes(p)
    packed = torch.empty(pkb, dtype=torch.uint8, device=dev)
    R.rkv_pack_decoder(p, d_wd, packed, pkb, stream)

    def call_packed():
        R.rkv_restore_packed(p, out.codes, out.scale, out.zmin, out.ref_idx, kv, packed, pkb, idx,
                             n, cfg.rope_theta, rout, "bf16", ws, wsb, stream)

    def call_repack():
        R.rkv_restore(p, out.codes, out.scale, out.zmin, out.ref_idx, kv, d_wd, idx, n,
                      cfg.rope_theta, rout, "bf16", ws, wsb, stream)

    def timed(call):
        for _ in range(max(args.warmup, 1)):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_repack = timed(call_repack)
    ms = timed(call_packed)
    st = R.STAGES.index("restore")
    R.rkv_profile_begin(1 << st)
    for _ in range(args.steps):
        call_packed()
    torch.cuda.synchronize()
    tot, cnt = R.rkv_profile_read(st)
    R.rkv_profile_begin(0)
    flops = 2.0 * n * cfg.d_c * cfg.C           # z~ W_d, the method's product
    return {"rows": n, "call": "rkv_restore_packed (W_d packed once by rkv_pack_decoder)",
            "ms_per_call": round(ms, 4), "rows_per_s": round(n / (ms * 1e-3), 1),
            "ms_per_call_rkv_restore_repacking": round(ms_repack, 4),
            "stage_ms": round(tot / cnt, 4),
            "decoder_tflops_algorithmic": round(flops / (tot / cnt * 1e-3) / 1e12, 2),
            "out_dtype": "bf16", "rope_theta": cfg.rope_theta}


def bench_append(R, cfg, p_enc, kv, w1, w2, w3, stream, args, batches=(1, 16)):
    """rkv_append ([RKV] §2.7 decode step 4) at the end of the workload's
    context: B sequences each append the token at a non-reference position
    near T, against a pool of every reference before it.  The cache of B
    sequences repeats the workload's sequence 0 (same shape and statistics);
    timed with events over repeated calls (each call rewrites the same
    records).  HBM bytes per call are algorithmic: the pool rows read by the
    distances, the chosen rows of the mean, the new rows, W1, W2 and W3 once,
    and the records written.  The same calls through rkv_append_proj (the
    cache's reference projections computed once beforehand) are timed
    beside them ("proj")."""
    import numpy as np
    import torch
    dev = kv.device
    refs = R.rkv_reference_positions(p_enc)
    mask = np.zeros(cfg.T, dtype=bool)
    mask[refs] = True
    nonref = np.flatnonzero(~mask)
    esz = 2 if cfg.dtype == "bf16" else 4
    rec = cfg.d_c * cfg.b // 8 + 4 * (cfg.d_c // cfg.g) + 4 * cfg.k
    out = []
    for B in batches:
        p = R.params(B=B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k, g=cfg.g,
                     b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
                     ref_alpha=cfg.alpha)
        cache = kv[:1].expand(B, -1, -1).contiguous()
        pos_h = nonref[len(nonref) - 1 - 3 * np.arange(B)]
        pos = torch.from_numpy(pos_h.astype(np.int32)).to(dev)
        kv_new = cache[torch.arange(B, device=dev), pos.long()].contiguous()
        n = B * cfg.T
        ref_idx = torch.empty((n, cfg.k), dtype=torch.int32, device=dev)
        codes = torch.empty((n, cfg.d_c * cfg.b // 8), dtype=torch.uint8, device=dev)
        scale = torch.empty((n, cfg.d_c // cfg.g), dtype=torch.float16, device=dev)
        zmin = torch.empty_like(scale)
        wsb = R.rkv_append_workspace_bytes(p)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def call():
            R.rkv_append(p, cache, kv_new, pos, w1, w2, w3, ref_idx, codes, scale, zmin, None, ws,
                         wsb, stream)

        for _ in range(max(args.warmup, 3)):
            call()
        st = R.STAGES.index("append")
        reps = max(args.steps, 50)
        # per call: back-to-back calls between two events, without the stage
        # profiler (its event pair per call costs host time that a call this
        # short would otherwise wait on); then the library's own stage events
        # in a second pass
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        R.rkv_profile_begin(1 << st)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        tot, cnt = R.rkv_profile_read(st)
        R.rkv_profile_begin(0)
        # the same call through rkv_append_proj, with the references'
        # projections of the cache computed once beforehand (rkv_project_refs)
        wsp = R.rkv_append_proj_workspace_bytes(p)
        wsp_t = torch.empty(wsp, dtype=torch.uint8, device=dev)
        ref_proj = torch.empty(R.rkv_ref_proj_bytes(p) // 4, dtype=torch.float32, device=dev)
        wpr = R.rkv_project_refs_workspace_bytes(p)
        wpr_t = torch.empty(wpr, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        R.rkv_project_refs(p, cache, w1, w2, ref_proj, wpr_t, wpr, stream)
        torch.cuda.synchronize()
        project_ms = (time.perf_counter() - t0) * 1e3
        del wpr_t

        def call_proj():
            R.rkv_append_proj(p, cache, ref_proj, kv_new, pos, w1, w2, w3, ref_idx, codes, scale,
                              zmin, None, wsp_t, wsp, stream)

        for _ in range(max(args.warmup, 3)):
            call_proj()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            call_proj()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_proj = e0.elapsed_time(e1) / reps
        R.rkv_profile_begin(1 << st)
        for _ in range(reps):
            call_proj()
        torch.cuda.synchronize()
        tot_p, cnt_p = R.rkv_profile_read(st)
        R.rkv_profile_begin(0)
        pools = np.searchsorted(np.asarray(refs), pos_h)          # references before each position
        nbytes = (int(pools.sum()) * cfg.C * esz + B * (cfg.k + 1) * cfg.C * esz
                  + (2 * cfg.C * cfg.d_ff + cfg.d_ff * cfg.d_c) * esz + B * rec)
        us = ms * 1e3
        out.append({"B": B, "us_per_call": round(us, 2), "tokens_per_s": round(B / (ms * 1e-3), 1),
                    "stage_us": round(tot / cnt * 1e3, 2), "hbm_bytes_algorithmic": nbytes,
                    "hbm_gb_s": round(nbytes / (tot / cnt * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (tot / cnt * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "pool_refs": int(pools.max()),
                    "proj": {"call": "rkv_append_proj (reference projections kept with the cache)",
                             "us_per_call": round(ms_proj * 1e3, 2),
                             "tokens_per_s": round(B / (ms_proj * 1e-3), 1),
                             "stage_us": round(tot_p / cnt_p * 1e3, 2),
                             "project_refs_ms_once": round(project_ms, 3)}})
        del cache, kv_new, ref_idx, codes, scale, zmin, ws, wsp_t, ref_proj
    return out


def bench_variants(R, RB, cfg, kv, w1, w2, w3, idx, stream, args):
    """The same step (encode + gather of the workload) with the references
    kept in FP8 ([RKV] §2.4 last paragraph) and with quantisation off
    (identity, b = 16), each timed like the main line."""
    import torch
    out = {}
    for name, kw in (("fp8_refs", dict(ref_format="fp8")), ("identity", dict(b=16))):
        d = dict(B=cfg.B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k, g=cfg.g,
                 b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
                 ref_alpha=cfg.alpha)
        d.update(kw)
        p = R.params(**d)
        buf = RB.alloc_encode(p, kv.device, with_z=False)
        gdst = torch.empty((idx.numel(), cfg.d_c), dtype=torch.bfloat16, device=kv.device)

        packed = RB.pack_weights(p, w1, w2, w3, stream)

        def step():
            RB.encode_packed(p, kv, packed, buf, stream)
            RB.dequant_gather(p, buf, idx, "bf16", stream, dst=gdst)

        for _ in range(max(args.warmup, 1)):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        out[name] = {"ms_per_step": round(ms, 4),
                     "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1)}
        del buf, gdst
    return out


def bench_vendor_gemm(cfg, refs, dev, reps: int = 20):
    """hipBLASLt (torch.matmul, bf16 in, fp32 accumulate) on the plain dense
    product of each contraction shape of the workload: the rate the vendor
    library reaches on that shape, and the encode's matrix-core time if every
    contraction ran at that rate with no epilogue, no top-k scan and no
    launch between them (the algorithmic flops of each stage over the
    library's rate for its shape; the causal distance work at the rate of the
    full token x reference product).  A reference point for the kernels, not
    a path of the library."""
    import torch
    nref, nr, pairs = schedule_counts(refs, cfg.T)
    B, C = cfg.B, cfg.C
    shapes = {  # stage: (M, N, K, algorithmic flops of the stage)
        "dist": (B * nr, nref, C, 2.0 * C * pairs * B),
        "proj": (B * nref, 2 * cfg.d_ff, C, 2.0 * C * 2 * cfg.d_ff * B * nref),
        "swiglu": (B * nr, 2 * cfg.d_ff, C, 2.0 * C * 2 * cfg.d_ff * B * nr),
        "w3": (B * nr, cfg.d_c, cfg.d_ff, 2.0 * cfg.d_ff * cfg.d_c * B * nr),
    }
    out, total_ms = {}, 0.0
    best = {}
    for _ in range(2):                 # two passes over the shapes; the faster of each counts
        for name, (m, n, k, work) in shapes.items():
            a = torch.randn((m, k), device=dev).to(torch.bfloat16)
            b = torch.randn((k, n), device=dev).to(torch.bfloat16)
            for _ in range(10):
                c = a @ b
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best.get(name, float("inf")), e0.elapsed_time(e1) / reps)
            del a, b, c
    for name, (m, n, k, work) in shapes.items():
        ms = best[name]
        rate = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        stage_ms = work / (rate * 1e12) * 1e3
        total_ms += stage_ms
        out[name] = {"m": m, "n": n, "k": k, "ms": round(ms, 4), "tflops": round(rate, 1),
                     "stage_ms_at_this_rate": round(stage_ms, 4)}
    mfma = sum(v[3] for v in shapes.values())
    out["encode_mfma_ms_at_vendor_rates"] = round(total_ms, 4)
    out["pct_bf16_peak_at_vendor_rates"] = round(
        100.0 * mfma / (total_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)
    return out


STAGE_PASS_STEPS = 20   # untimed steps with every stage bracketed (the stage breakdown)
FLUSH_MB = 512          # written before every cold gather call: twice the 256 MB MALL


def bench_gather_cold(R, RB, cfg, p, out, idx, stream, reps: int = 20):
    """rkv_dequant_gather of the workload's rows with cold caches: before
    every timed call a 512 MB buffer is written (evicting the 256 MB MALL and
    every L2), then the call alone is bracketed by events; median of `reps`.
    GB/s counts the algorithmic bytes (each row's record read, its bf16 row
    written).  The launch floor is the same measurement for a single row."""
    import numpy as np
    import torch
    dev = idx.device
    flush = torch.empty(FLUSH_MB << 20, dtype=torch.uint8, device=dev)
    rec = cfg.d_c * cfg.b // 8 + (0 if cfg.b == 16 else 4 * (cfg.d_c // cfg.g))

    def timed(ix):
        dst = torch.empty((ix.numel(), cfg.d_c), dtype=torch.bfloat16, device=dev)
        ms = []
        for i in range(reps + 2):
            flush.fill_(i & 0xFF)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            RB.dequant_gather(p, out, ix, "bf16", stream, dst=dst)
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    ms = timed(idx)
    floor = timed(idx[:1])
    nbytes = idx.numel() * (rec + 2 * cfg.d_c)
    del flush
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"rows": int(idx.numel()), "bytes_algorithmic": int(nbytes), "us": round(ms * 1e3, 2),
            "gb_s": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "launch_floor_us": round(floor * 1e3, 2),
            "gb_s_above_floor": round(nbytes / (max(ms - floor, 1e-6) * 1e-3) / 1e9, 1),
            "flush_mb": FLUSH_MB, "reps": reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clocks after a few tens of steps (about
    # 7% faster than right after start): warm up past that by default
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama8b_T32k")
    ap.add_argument("--cpu-tokens", type=int, default=4096)   # about 15 s of oracle work
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the append measurement")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the FP8-reference and identity-mode encode measurements")
    ap.add_argument("--no-restore", action="store_true",
                    help="skip the separate restore measurement (rkv_restore of the gathered rows)")
    ap.add_argument("--copy-check-mb", type=int, default=0,
                    help="before the timed region, run one plain device copy of this many MiB "
                         "(a reference of known size for hardware byte counters)")
    ap.add_argument("--mfma-check", type=int, default=0,
                    help="before the timed region, run one torch bf16 matmul of this size "
                         "(n x n times n x n, 2 n^3 flops): a reference of known work for the "
                         "matrix-core op counters")
    ap.add_argument("--no-gather-cold", action="store_true",
                    help="skip the cold-cache gather measurement")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time hipBLASLt (torch.matmul) on the plain product of each "
                         "contraction shape, as a reference point for the kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: librkv has no multi-GPU path (the encode "
              "would shard by sequence or by token range, with the reference rows exchanged "
              "once).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import reference_residual_encoding_amd as R
    from reference_residual_encoding_amd import buffers as RB
    from synth import config_by_name, generate

    cfg = config_by_name(args.workload)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    w = generate(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    p = R.params(B=cfg.B, T=cfg.T, N=cfg.N, D=cfg.D, d_ff=cfg.d_ff, d_c=cfg.d_c, k=cfg.k,
                 g=cfg.g, b=cfg.b, ref_stride=cfg.stride, dtype=cfg.dtype, n_sink=cfg.n_sink,
                 ref_alpha=cfg.alpha)
    kv, w1, w2, w3 = (to_dev(x) for x in (w.kv, w.w1, w.w2, w.w3))
    out = RB.alloc_encode(p, dev, with_z=False)
    idx = torch.from_numpy(w.gather_idx.astype(np.int32)).to(dev)
    gdst = torch.empty((idx.numel(), cfg.d_c), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    # the compressor's weights are constants of the trained codec: packed
    # once into the operand layout of the matrix-core products, as a
    # deployment does when it loads the model
    packed = RB.pack_weights(p, w1, w2, w3, stream)

    def step():
        RB.encode_packed(p, kv, packed, out, stream)
        RB.dequant_gather(p, out, idx, "bf16", stream, dst=gdst)

    def step_repack():                                   # rkv_encode: repacks at every call
        RB.encode(p, kv, w1, w2, w3, out, stream)
        RB.dequant_gather(p, out, idx, "bf16", stream, dst=gdst)

    if args.copy_check_mb:
        src = torch.empty(args.copy_check_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.mfma_check:
        n = args.mfma_check
        a = torch.ones((n, n), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        c = a @ a
        torch.cuda.synchronize()
        del a, c
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    # a short pass with every stage bracketed by events: the stage breakdown
    # and the dominant kernel
    R.rkv_profile_begin((1 << len(R.STAGES)) - 1)
    for _ in range(STAGE_PASS_STEPS):
        step()
    torch.cuda.synchronize()
    stages_ms = {}
    for i, name in enumerate(R.STAGES):
        tot, n = R.rkv_profile_read(i)
        if n:
            stages_ms[name] = tot / n
    dominant = max(stages_ms, key=stages_ms.get)
    dom_i = R.STAGES.index(dominant)
    print(f"[bench] stage ms: { {k: round(v, 4) for k, v in stages_ms.items()} }",
          file=sys.stderr, flush=True)

    def timed_steps(fn=step):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # timed region: K whole steps, no event inside a step
    R.rkv_profile_begin(0)
    ms_per_step = timed_steps()
    # the same K steps again, now with the dominant stage bracketed by an
    # event pair on the stream its kernel runs on: its launch duration
    R.rkv_profile_begin(1 << dom_i)
    ms_per_step_bracketed = timed_steps()
    dom_total, dom_n = R.rkv_profile_read(dom_i)
    R.rkv_profile_begin(0)
    dom_ms = dom_total / dom_n
    # the same step through rkv_encode, which repacks the weights at every call
    for _ in range(5):
        step_repack()
    ms_per_step_repack = timed_steps(step_repack)

    work = stage_work(cfg, idx.numel(), R.rkv_reference_positions(p))
    kind, amount = work[dominant]
    traffic = measured_traffic(cfg.name, STAGE_KERNEL[dominant])
    if kind == "flops":
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = amount / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dominant,
                "kernel_ms": round(dom_ms, 4), "work_per_launch": amount}
    else:
        achieved = amount / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": dominant, "kernel_ms": round(dom_ms, 4), "work_per_launch": amount}

    mfma_flops = sum(work[s][1] for s in ("dist", "swiglu", "w3"))
    encode_ms = sum(v for k, v in stages_ms.items() if k != "gather")
    tokens = cfg.B * cfg.T
    line = {
        "metric": "KV tokens encoded/sec (Llama-3.1-8B layer shape, T=32k); % bf16 MFMA peak",
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "N": cfg.N, "D": cfg.D,
                   "C": cfg.C, "d_ff": cfg.d_ff, "d_c": cfg.d_c, "k": cfg.k, "g": cfg.g,
                   "b": cfg.b, "ref_stride": cfg.stride, "ref_alpha": cfg.alpha, "n_sink": cfg.n_sink,
                   "gather_rows": int(idx.numel())},
        "pct_bf16_mfma_peak": round(100.0 * mfma_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "encode_mfma_tflop_per_step": round(mfma_flops / 1e12, 4),
        "encode_mfma_tflops_achieved": round(mfma_flops / (ms_per_step * 1e-3) / 1e12, 1),
        "non_reference_tokens_per_s": round(cfg.B * schedule_counts(R.rkv_reference_positions(p), cfg.T)[1]
                                            / (ms_per_step * 1e-3), 1),
        "ms_per_step_with_kernel_events": round(ms_per_step_bracketed, 4),
        "encode_call": "rkv_encode_packed (weights packed once by rkv_pack_weights)",
        "ms_per_step_rkv_encode_repacking": round(ms_per_step_repack, 4),
        "stages_ms": {k: round(v, 4) for k, v in stages_ms.items()},
        "encode_ms_stage_sum": round(encode_ms, 4),
        "roofline": roof,
    }
    if not args.no_gather_cold:
        line["gather"] = bench_gather_cold(R, RB, cfg, p, out, idx, stream)
    if not args.no_restore:
        line["restore"] = bench_restore(R, cfg, w, p, kv, out, idx, stream, args)
    if not args.no_append:
        line["append"] = bench_append(R, cfg, p, kv, w1, w2, w3, stream, args)
    if not args.no_variants:
        line["variants"] = bench_variants(R, RB, cfg, kv, w1, w2, w3, idx, stream, args)
    if args.vendor_gemm:
        line["vendor_gemm"] = bench_vendor_gemm(cfg, R.rkv_reference_positions(p), dev)
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
