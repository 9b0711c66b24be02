"""Workload shapes and seeded synthetic inputs.

This module only names shapes and draws random numbers; it holds none of the attention
arithmetic, so both the GPU path's callers and the CPU oracle's callers can share it.

Shapes come from the pages' models: the Llama-3-8B attention layer (32 query heads over 8
K/V heads, head_dim 128; llama3-from-scratch page, "model configuration parameters"), the
PaLM multi-query default (8 heads of dim 64 sharing one K/V head, batch 8, sequence 1024;
PaLM page, sections 2.5 and 4), a SmolLM-1.7B-shaped MHA layer at Picotron's micro-batch 4
and sequence 1024 (Picotron page, "configuration and usage"), a 32K-token single-GPU
shard of a sequence-parallel run (Megatron-DeepSpeed page, "32K long-sequence training"), and
the head size 256 of PaLM's 540B configuration (PaLM page, section 3).
The pages train on text corpora that are not available here; attention inputs are the
projected q/k/v activations, so seeded Gaussians of the same shapes stand in for them.

Recipe: torch.Generator('cpu').manual_seed(seed); draw q, then k, then v with
torch.randn(shape, dtype=float32) * sigma; cast to bfloat16 (round-to-nearest-even) unless
the workload is float32.  The same tensors feed the GPU and (as float64) the oracle.
"""

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    d: int
    dtype: str  # "bf16" or "fp32"
    sigma: float
    rope_theta: float
    causal: bool
    seed: int

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny_mqa_fp32": Workload("tiny_mqa_fp32", 1, 64, 4, 1, 64, "fp32", 1.0, 10000.0, True, 1),
    "llama3_8b": Workload("llama3_8b", 1, 2048, 32, 8, 128, "bf16", 1.0, 500000.0, True, 2),
    "palm_mqa": Workload("palm_mqa", 8, 1024, 8, 1, 64, "bf16", 1.0, 10000.0, True, 3),
    "smollm_mha": Workload("smollm_mha", 4, 1024, 32, 32, 64, "bf16", 0.5, 10000.0, True, 4),
    "long_shard": Workload("long_shard", 1, 32768, 32, 8, 128, "bf16", 1.0, 500000.0, True, 5),
    # head size of the PaLM page's largest configuration (section 3: 48 heads of 256, one
    # shared K/V head) at the page's example sequence length
    "palm540b_d256": Workload("palm540b_d256", 1, 2048, 48, 1, 256, "bf16", 1.0, 10000.0, True, 6),
}

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def make_inputs(w: Workload):
    """Seeded (q, k, v) CPU tensors in the workload's dtype, drawn in the order q, k, v."""
    g = torch.Generator(device="cpu").manual_seed(int(w.seed))
    q = torch.randn((w.B, w.S, w.Hq, w.d), dtype=torch.float32, generator=g) * w.sigma
    k = torch.randn((w.B, w.S, w.Hkv, w.d), dtype=torch.float32, generator=g) * w.sigma
    v = torch.randn((w.B, w.S, w.Hkv, w.d), dtype=torch.float32, generator=g) * w.sigma
    dt = TORCH_DTYPE[w.dtype]
    return q.to(dt), k.to(dt), v.to(dt)
