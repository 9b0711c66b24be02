"""Fused causal RoPE + grouped-query attention forward for AMD MI355X (gfx950).

    out, lse = attn_fwd(q, k, v, rope_theta, causal=True)

q: (B, S, Hq, D), k/v: (B, S, Hkv, D) contiguous CUDA (HIP) tensors, bfloat16 or float32,
D in {64, 128}, Hq a multiple of Hkv.  Returns out (B, S, Hq, D) in the input dtype and
lse (B, Hq, S) float32 (natural-log logsumexp of the scaled scores of each row).

    out, lse = attn_fwd(q, k, v, rope_theta, causal=True, q_pos0=p, k_pos0=r)
    out, lse = attn_merge(o1, lse1, o2, lse2)

A call with position offsets is one shard of a longer sequence (one ring-attention step);
attn_merge joins two such partial results.

    cache = new_kv_cache(B, S_cap, Hkv, D, device)
    kv_prepare(k, v, rope_theta, key0, key1, cache)
    out, lse = attn_decode(q, cache, S_cap, Hkv, rope_theta, q_pos)

is the decode step: one query per (batch row, head) at position q_pos over the cached keys
0 .. q_pos (bf16); kv_prepare rotates and stores keys as they are appended.

    dq, dk, dv = attn_bwd(q, k, v, out, lse, dout, rope_theta, causal=True)

is the backward pass (bf16), from the forward's out and lse.

PyTorch only provides device memory and the stream; the computation runs in the HIP
kernels behind the C ABI of libattn.so (include/attn.h).
"""

from ._lib import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_FP32,
    AttnError,
    Event,
    abi_version,
    load,
    strerror,
    bwd_workspace_bytes,
    decode_workspace_bytes,
    workspace_bytes,
)
from .api import (  # noqa: F401
    attn_bwd,
    attn_decode,
    attn_fwd,
    attn_fwd_into,
    attn_fwd_noalloc,
    attn_merge,
    kv_cache_bytes,
    kv_prepare,
    new_kv_cache,
)
