"""The five synthetic workloads of the ResidualKV cache-write path.

Notation follows the ResidualKV reading notes (arXiv 2602.08005v2), §2.1
symbol table: B sequences of T tokens, N KV heads of dimension D, so that
2*d_k = 2*N*D coordinates per joint [K|V] token vector; compressor width d_ff;
latent width d_c; k neighbours; quantiser group g and bit width b (§2.4); a
reference every ``stride`` tokens (§2.6, fixed-stride schedule).

The shapes borrow 2*d_k from the notes' §3.1 model table (Llama-3.1-8B: 2048;
Qwen2.5-7B: 1024).  d_ff, d_c and the stride are the workload's own choices.
"""
from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class RkvConfig:
    name: str
    B: int
    T: int
    N: int
    D: int
    d_ff: int
    d_c: int
    k: int
    g: int
    b: int
    stride: int
    dtype: str                 # "f32" or "bf16": dtype of kv and of W1..W3
    kind: str                  # data recipe: "proto", "proto_t4", "multimodal"
    n_protos: int = 0          # prototypes of the clustered recipes
    noise: float = 0.0         # noise scale of the clustered recipes
    gather_frac: Optional[float] = None  # None: gather every position
    seed: int = 0
    rope_theta: float = 10000.0  # RoPE base of the model whose keys are restored
    alpha: float = 0.0         # reference schedule growth ([RKV] §2.6); 0 = fixed stride
    n_sink: int = 0            # sink tokens, stored as references before the schedule starts
    ref_fp8: bool = False      # references stored as FP8 E4M3 ([RKV] §2.4 last paragraph)
    # multimodal recipe only
    mm_blocks: int = 0
    mm_block_len: int = 0
    mm_block_protos: int = 0
    mm_image_noise: float = 0.0
    mm_text_protos: int = 0
    mm_text_noise: float = 0.0
    mm_run_min: int = 0
    mm_run_max: int = 0

    @property
    def C(self) -> int:
        """Joint vector width 2*d_k = 2*N*D."""
        return 2 * self.N * self.D

    def with_(self, **kw) -> "RkvConfig":
        return dataclasses.replace(self, **kw)


TINY = RkvConfig(
    name="tiny_f32", B=1, T=256, N=2, D=16, d_ff=64, d_c=32, k=4, g=32, b=4,
    stride=8, dtype="f32", kind="proto", n_protos=16, noise=0.3)

LLAMA8K = RkvConfig(
    name="llama8b_T8k", B=1, T=8192, N=8, D=128, d_ff=1024, d_c=512, k=4, g=32,
    b=4, stride=16, dtype="bf16", kind="proto", n_protos=256, noise=0.25,
    rope_theta=500000.0)

LLAMA32K = LLAMA8K.with_(name="llama8b_T32k", T=32768, gather_frac=0.30)

QWEN_LIKE = RkvConfig(
    name="qwen7b_like_B2_T32k", B=2, T=32768, N=4, D=128, d_ff=512, d_c=256,
    k=4, g=32, b=4, stride=16, dtype="bf16", kind="proto_t4", n_protos=512,
    noise=0.25, rope_theta=1000000.0)

MM_INT2 = RkvConfig(
    name="multimodal_int2_B4_T16k", B=4, T=16384, N=8, D=128, d_ff=1024,
    d_c=512, k=4, g=32, b=2, stride=16, dtype="bf16", kind="multimodal",
    gather_frac=0.10, mm_blocks=24, mm_block_len=576, mm_block_protos=32,
    mm_image_noise=0.2, mm_text_protos=256, mm_text_noise=0.4, mm_run_min=32,
    mm_run_max=128, rope_theta=500000.0)

CONFIGS = [TINY, LLAMA8K, LLAMA32K, QWEN_LIKE, MM_INT2]




# Dynamic reference schedules ([RKV] §2.6, the notes' LongBench setting
# alpha = 0.001 with the default initial stride 10): parity and measurement
# cases beside the five fixed-stride workloads above.
TINY_DYN = TINY.with_(name="tiny_f32_dynamic", alpha=0.02, n_sink=2)
LLAMA8K_DYN = LLAMA8K.with_(name="llama8b_T8k_dynamic", stride=10, alpha=0.001, n_sink=4)
LLAMA32K_DYN = LLAMA32K.with_(name="llama8b_T32k_dynamic", stride=10, alpha=0.001, n_sink=4)
DYNAMIC = (TINY_DYN, LLAMA8K_DYN, LLAMA32K_DYN)


def config_by_name(name: str) -> RkvConfig:
    for c in list(CONFIGS) + list(DYNAMIC):
        if c.name == name:
            return c
    raise KeyError(name)
