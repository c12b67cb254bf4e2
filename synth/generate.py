"""Seeded generators for the synthetic ResidualKV workloads.

Why clustered data: the ResidualKV notes (§1.2, observations on Fig. 3) report
that a token's best historical match has high cosine similarity (mean 0.92)
and is often far away (most best matches sit more than 16 positions back).
Prototype-plus-noise vectors with a uniform prototype assignment reproduce
both traits: same-prototype cosine is 1/(1+sigma^2) (0.94 at sigma=0.25,
0.92 at 0.3) and a token's nearest same-prototype reference lies anywhere in
the history.

Draw order (one ``numpy.random.default_rng(seed)`` stream, fixed so that every
consumer reproduces the same bits):
  clustered recipes: prototypes -> assignments -> noise -> W1 -> W2 -> W3 ->
                     gather indices
  multimodal recipe: text prototypes -> per-sequence run lengths ->
                     per-block image prototypes -> assignments -> noise ->
                     W1 -> W2 -> W3 -> gather indices
All draws are float32; bf16 workloads are then rounded to bf16
(round-to-nearest-even) once, and those bits are what both sides consume.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from .configs import RkvConfig


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    cfg: RkvConfig
    kv: np.ndarray          # [B,T,C]  float32 (f32) or uint16 bf16 bits (bf16)
    w1: np.ndarray          # [C,d_ff]
    w2: np.ndarray          # [C,d_ff]
    w3: np.ndarray          # [d_ff,d_c]
    gather_idx: np.ndarray  # int32 flat b*T+t, sorted ascending
    segments: Optional[List[List[Tuple[str, int, int]]]] = None  # multimodal layout

    def _widen(self, a: np.ndarray) -> np.ndarray:
        if self.cfg.dtype == "bf16":
            return bf16_bits_to_f32(a)
        return np.asarray(a, dtype=np.float32)

    def kv_f32(self) -> np.ndarray:
        return self._widen(self.kv)

    def weights_f32(self):
        return self._widen(self.w1), self._widen(self.w2), self._widen(self.w3)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _weights(rng, cfg: RkvConfig):
    C = cfg.C
    w1 = rng.standard_normal((C, cfg.d_ff), dtype=np.float32) * np.float32(1.0 / np.sqrt(C))
    w2 = rng.standard_normal((C, cfg.d_ff), dtype=np.float32) * np.float32(1.0 / np.sqrt(C))
    w3 = rng.standard_normal((cfg.d_ff, cfg.d_c), dtype=np.float32) * np.float32(1.0 / np.sqrt(cfg.d_ff))
    return w1, w2, w3


def _gather(rng, cfg: RkvConfig) -> np.ndarray:
    total = cfg.B * cfg.T
    if cfg.gather_frac is None:
        return np.arange(total, dtype=np.int32)
    n = int(np.floor(cfg.gather_frac * total))
    idx = rng.choice(total, size=n, replace=False)
    return np.sort(idx).astype(np.int32)


def _multimodal_layout(rng, cfg: RkvConfig):
    """Text run, image block, text run, image block ... then text to the end.

    Run lengths are uniform integers in [run_min, run_max]; everything is
    truncated at T.
    """
    T = cfg.T
    segs: List[Tuple[str, int, int]] = []
    pos = 0
    for _ in range(cfg.mm_blocks):
        if pos >= T:
            break
        L = int(rng.integers(cfg.mm_run_min, cfg.mm_run_max + 1))
        segs.append(("text", pos, min(pos + L, T)))
        pos += L
        if pos >= T:
            break
        segs.append(("image", pos, min(pos + cfg.mm_block_len, T)))
        pos += cfg.mm_block_len
    while pos < T:
        L = int(rng.integers(cfg.mm_run_min, cfg.mm_run_max + 1))
        segs.append(("text", pos, min(pos + L, T)))
        pos += L
    return segs


def generate(cfg: RkvConfig) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    B, T, C = cfg.B, cfg.T, cfg.C
    segments = None
    if cfg.kind in ("proto", "proto_t4"):
        protos = rng.standard_normal((cfg.n_protos, C), dtype=np.float32)
        assign = rng.integers(0, cfg.n_protos, size=(B, T))
        if cfg.kind == "proto":
            noise = rng.standard_normal((B, T, C), dtype=np.float32)
        else:
            noise = rng.standard_t(4, size=(B, T, C)).astype(np.float32)
        noise *= np.float32(cfg.noise)
        noise += protos[assign]
        kv = noise
    elif cfg.kind == "multimodal":
        text_protos = rng.standard_normal((cfg.mm_text_protos, C), dtype=np.float32)
        segments = [_multimodal_layout(rng, cfg) for _ in range(B)]
        image_protos = [[rng.standard_normal((cfg.mm_block_protos, C), dtype=np.float32)
                         for (kind, _, _) in segs if kind == "image"]
                        for segs in segments]
        kv = np.empty((B, T, C), dtype=np.float32)
        scale = np.empty((B, T, 1), dtype=np.float32)
        for bi, segs in enumerate(segments):
            blk = 0
            for kind, a, e in segs:
                if kind == "text":
                    c = rng.integers(0, cfg.mm_text_protos, size=e - a)
                    kv[bi, a:e] = text_protos[c]
                    scale[bi, a:e] = cfg.mm_text_noise
                else:
                    c = rng.integers(0, cfg.mm_block_protos, size=e - a)
                    kv[bi, a:e] = image_protos[bi][blk][c]
                    scale[bi, a:e] = cfg.mm_image_noise
                    blk += 1
        for bi in range(B):
            kv[bi] += rng.standard_normal((T, C), dtype=np.float32) * scale[bi]
    else:
        raise ValueError(f"unknown recipe {cfg.kind}")
    w1, w2, w3 = _weights(rng, cfg)
    gidx = _gather(rng, cfg)
    return Workload(cfg=cfg, kv=_finish(kv, cfg.dtype), w1=_finish(w1, cfg.dtype),
                    w2=_finish(w2, cfg.dtype), w3=_finish(w3, cfg.dtype),
                    gather_idx=gidx, segments=segments)


def decoder_weight(cfg: RkvConfig) -> np.ndarray:
    """W_d [d_c][C] of the linear restore map z -> z W_d, N(0, 1/d_c).

    Drawn from its own stream, ``default_rng((seed, 1))``, so the encode
    workloads above keep their draws.  Rounded to bf16 for bf16 workloads
    (uint16 bits), float32 otherwise."""
    rng = np.random.default_rng((cfg.seed, 1))
    wd = rng.standard_normal((cfg.d_c, cfg.C), dtype=np.float32) * np.float32(1.0 / np.sqrt(cfg.d_c))
    return _finish(wd, cfg.dtype)
