"""Device buffers for librkv calls, allocated with PyTorch (plumbing only).

Shapes follow include/rkv.h.  scale/zmin are float16 tensors holding the
fp16 Delta_h and m_h; ref_idx is int32; codes are uint8.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (RKV_BF16, RKV_F32, rkv_dequant_gather, rkv_encode, rkv_encode_packed,
               rkv_encode_workspace_bytes, rkv_pack_weights, rkv_packed_weights_bytes, rkv_params)


@dataclasses.dataclass
class EncodeBuffers:
    ref_idx: torch.Tensor
    codes: torch.Tensor
    scale: torch.Tensor
    zmin: torch.Tensor
    z: Optional[torch.Tensor]
    workspace: torch.Tensor


def alloc_encode(p: rkv_params, device="cuda", with_z: bool = True) -> EncodeBuffers:
    B, T = p.B, p.T
    ng = 0 if p.b == 16 else p.d_c // p.g          # identity mode stores no group numbers
    ws = rkv_encode_workspace_bytes(p)
    if ws == 0:
        raise ValueError("invalid rkv_params")
    return EncodeBuffers(
        ref_idx=torch.empty((B, T, p.k), dtype=torch.int32, device=device),
        codes=torch.empty((B, T, p.d_c * p.b // 8), dtype=torch.uint8, device=device),
        scale=torch.empty((B, T, ng), dtype=torch.float16, device=device),
        zmin=torch.empty((B, T, ng), dtype=torch.float16, device=device),
        z=torch.empty((B, T, p.d_c), dtype=torch.float32, device=device) if with_z else None,
        workspace=torch.empty(ws, dtype=torch.uint8, device=device),
    )


def encode(p: rkv_params, kv, w1, w2, w3, out: EncodeBuffers, stream=None) -> EncodeBuffers:
    if stream is None:
        stream = torch.cuda.current_stream(kv.device)
    rkv_encode(p, kv, w1, w2, w3, out.ref_idx, out.codes, out.scale, out.zmin, out.z,
               out.workspace, out.workspace.numel(), stream)
    return out


def pack_weights(p: rkv_params, w1, w2, w3, stream=None) -> torch.Tensor:
    """The compressor weights in the encode's operand layout (pack once,
    encode many times with encode_packed)."""
    n = rkv_packed_weights_bytes(p)
    if n == 0:
        raise ValueError("invalid rkv_params")
    packed = torch.empty(n, dtype=torch.uint8, device=w1.device)
    if stream is None:
        stream = torch.cuda.current_stream(w1.device)
    rkv_pack_weights(p, w1, w2, w3, packed, n, stream)
    return packed


def encode_packed(p: rkv_params, kv, packed: torch.Tensor, out: EncodeBuffers,
                  stream=None) -> EncodeBuffers:
    if stream is None:
        stream = torch.cuda.current_stream(kv.device)
    rkv_encode_packed(p, kv, packed, packed.numel(), out.ref_idx, out.codes, out.scale, out.zmin,
                      out.z, out.workspace, out.workspace.numel(), stream)
    return out


def dequant_gather(p: rkv_params, out: EncodeBuffers, idx: torch.Tensor, out_dtype="f32",
                   stream=None, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    code = {"f32": RKV_F32, "bf16": RKV_BF16}.get(out_dtype, out_dtype)
    if dst is None:
        dt = torch.float32 if code == RKV_F32 else torch.bfloat16
        dst = torch.empty((idx.numel(), p.d_c), dtype=dt, device=idx.device)
    if stream is None:
        stream = torch.cuda.current_stream(idx.device)
    rkv_dequant_gather(p, out.codes, out.scale, out.zmin, idx, idx.numel(), dst, code, stream)
    return dst
