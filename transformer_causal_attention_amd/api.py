"""PyTorch-facing wrapper of attn_fwd: checks tensors, allocates outputs, passes pointers."""

import torch

from . import _lib

_DTYPE_CODE = {torch.bfloat16: _lib.ATTN_DTYPE_BF16, torch.float32: _lib.ATTN_DTYPE_FP32}


def _shapes(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D tensor (B, S, H, D)")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype: bfloat16 or float32")
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError(f"k and v must be (B, S, Hkv, D) = ({B}, {S}, Hkv, {D}); got {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    return B, S, Hq, Hkv, D


def _keep_for(stream, *allocated):
    """Tensors this wrapper allocated on the current stream but hands to kernels on `stream`: record
    that stream on them, so the caching allocator does not reuse their memory (after the caller
    frees them) before those kernels are done."""
    if stream is not None:
        for t in allocated:
            if t is not None:
                t.record_stream(stream)


def _rope_style(interleaved):
    return _lib.ATTN_ROPE_INTERLEAVED if interleaved else _lib.ATTN_ROPE_HALF


def attn_fwd_into(q, k, v, rope_theta, causal, out, lse, workspace=None, stream=None, events=None,
                  q_pos0=0, k_pos0=0, interleaved=False):
    """attn_fwd writing into caller-provided out (like q) and lse (B, Hq, S) float32.

    workspace: optional uint8 GPU tensor of at least workspace_bytes(...) bytes.
    stream: torch.cuda.Stream to enqueue on (default: the current stream).
    events: optional (start, stop) pair of Event recorded around the attention kernel.
    q_pos0, k_pos0: positions of query row 0 and key row 0 when the call is one shard of a
    longer sequence (attn_fwd_shard); events are not available for shards.
    interleaved: rotate adjacent dim pairs (2i, 2i+1) instead of (i, i + D/2).
    """
    B, S, Hq, Hkv, D = _shapes(q, k, v)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if tuple(lse.shape) != (B, Hq, S) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, S)")
    code = _DTYPE_CODE[q.dtype]
    need = _lib.workspace_bytes(B, S, Hkv, D, code)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if stream is not None:
            workspace.record_stream(st)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if q_pos0 or k_pos0:
        if events is not None:
            raise ValueError("events are not available for a shard call")
        rc = _lib.shard_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, S, Hq, Hkv, D, rope_theta,
                            1 if causal else 0, q_pos0, k_pos0, code, out.data_ptr(), lse.data_ptr(),
                            ws_ptr, ws_bytes, st.cuda_stream, rope_style=_rope_style(interleaved))
        if rc != _lib.ATTN_OK:
            raise _lib.AttnError(rc, "attn_fwd_shard")
        return out, lse
    ev0, ev1 = (events[0].ptr, events[1].ptr) if events is not None else (None, None)
    rc = _lib.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, S, Hq, Hkv, D, rope_theta,
                      1 if causal else 0, code, out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes,
                      st.cuda_stream, ev0, ev1, rope_style=_rope_style(interleaved))
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_fwd")
    return out, lse


def attn_fwd(q, k, v, rope_theta, causal=True, workspace=None, stream=None, events=None, q_pos0=0, k_pos0=0,
             interleaved=False):
    """Fused RoPE + causal GQA attention forward.  Returns (out, lse).

    interleaved: adjacent-pair rotary form (dims 2i, 2i+1) instead of the half-split one.

    With q_pos0 / k_pos0 the call is one shard of a longer sequence (queries at q_pos0 + i,
    keys at k_pos0 + j); rows that see no key get out 0 and lse -inf, ready for attn_merge.
    """
    B, S, Hq, Hkv, D = _shapes(q, k, v)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _keep_for(stream, out, lse)
    return attn_fwd_into(q, k, v, rope_theta, causal, out, lse, workspace, stream, events, q_pos0, k_pos0,
                         interleaved)


def attn_fwd_noalloc(q, k, v, rope_theta, causal, out, lse, stream=None, interleaved=False):
    """attn_fwd through attn_fwd_noalloc: no workspace, and nothing allocated by this call.

    out (like q) and lse ((B, Hq, S) float32) are caller-provided; the library's own fixed
    scratch serves as workspace (calls that overlap in time on one GPU race on it).
    """
    B, S, Hq, Hkv, D = _shapes(q, k, v)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if tuple(lse.shape) != (B, Hq, S) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, S)")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = _lib.fwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, S, Hq, Hkv, D, rope_theta,
                              1 if causal else 0, _DTYPE_CODE[q.dtype], out.data_ptr(), lse.data_ptr(),
                              st.cuda_stream, rope_style=_rope_style(interleaved))
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_fwd_noalloc")
    return out, lse


def attn_merge(o1, lse1, o2, lse2, out=None, lse=None, stream=None):
    """Join two partial results over disjoint keys (attn_merge).  Returns (out, lse).

    o1, o2: (B, S, H, D) like attn_fwd's out; lse1, lse2: (B, H, S) float32.  out / lse may be
    given, and may be o1 / lse1 (in place).
    """
    for name, t in (("o1", o1), ("o2", o2)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor (B, S, H, D)")
    if o2.shape != o1.shape or o2.dtype != o1.dtype or o1.dtype not in _DTYPE_CODE:
        raise ValueError("o1 and o2 must share shape and a dtype of bfloat16 or float32")
    B, S, H, D = o1.shape
    for name, t in (("lse1", lse1), ("lse2", lse2)):
        if tuple(t.shape) != (B, H, S) or t.dtype != torch.float32 or not t.is_contiguous() or t.device != o1.device:
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape (B, H, S)")
    made = (torch.empty_like(o1) if out is None else None, torch.empty_like(lse1) if lse is None else None)
    out = made[0] if out is None else out
    lse = made[1] if lse is None else lse
    _keep_for(stream, *made)
    if out.shape != o1.shape or out.dtype != o1.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like o1")
    if lse.shape != lse1.shape or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor shaped like lse1")
    st = stream if stream is not None else torch.cuda.current_stream(o1.device)
    rc = _lib.merge_raw(o1.data_ptr(), lse1.data_ptr(), o2.data_ptr(), lse2.data_ptr(), B, S, H, D,
                        _DTYPE_CODE[o1.dtype], out.data_ptr(), lse.data_ptr(), st.cuda_stream)
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_merge")
    return out, lse


def _gpu_bf16(name, t, dims):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dims}-D GPU tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (the decode path is bf16 only)")


def kv_cache_bytes(B, S_cap, Hkv, head_dim):
    """Bytes of a decode key/value cache of capacity S_cap (rotated keys and transposed values)."""
    return _lib.workspace_bytes(B, S_cap, Hkv, head_dim, _lib.ATTN_DTYPE_BF16)


def new_kv_cache(B, S_cap, Hkv, head_dim, device):
    """An uninitialised cache (uint8 GPU tensor) for kv_prepare / attn_decode."""
    n = kv_cache_bytes(B, S_cap, Hkv, head_dim)
    if n == 0:
        raise ValueError("unsupported cache sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def kv_prepare(k, v, rope_theta, key0, key1, cache, stream=None, interleaved=False):
    """Rotate and store keys [key0, key1) of k (and their values) into cache (attn_kv_prepare).

    k, v: (B, S_cap, Hkv, D) bfloat16 holding valid rows from 64 * (key0 // 64) to key1.
    """
    _gpu_bf16("k", k, 4)
    _gpu_bf16("v", v, 4)
    if v.shape != k.shape or v.device != k.device:
        raise ValueError("k and v must share shape and device")
    if cache.dtype != torch.uint8 or cache.device != k.device or not cache.is_contiguous():
        raise ValueError("cache must be a contiguous uint8 tensor on k's device")
    B, S_cap, Hkv, D = k.shape
    st = stream if stream is not None else torch.cuda.current_stream(k.device)
    rc = _lib.kv_prepare_raw(k.data_ptr(), v.data_ptr(), B, S_cap, Hkv, D, rope_theta, key0, key1,
                             cache.data_ptr(), cache.numel(), st.cuda_stream, rope_style=_rope_style(interleaved))
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_kv_prepare")
    return cache


def attn_decode(q, cache, S_cap, Hkv, rope_theta, q_pos, out=None, lse=None, workspace=None, stream=None,
                interleaved=False, max_pos=None):
    """One decode step: q (B, Hq, D) bfloat16 at position q_pos against cached keys 0 .. q_pos.

    Returns (out (B, Hq, D) bfloat16, lse (B, Hq) float32), equal to row q_pos of attn_fwd.
    q_pos may also be an int32 GPU tensor of B positions, one per batch row (a ragged batch,
    attn_decode_ragged); max_pos bounds them (default S_cap - 1, which needs no host read of
    the positions but splits the keys for the longest possible row).
    """
    _gpu_bf16("q", q, 3)
    B, Hq, D = q.shape
    if cache.dtype != torch.uint8 or cache.device != q.device or not cache.is_contiguous():
        raise ValueError("cache must be a contiguous uint8 tensor on q's device")
    made = (torch.empty_like(q) if out is None else None,
            torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse is None else None)
    out = made[0] if out is None else out
    lse = made[1] if lse is None else lse
    _keep_for(stream, *made)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if tuple(lse.shape) != (B, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq)")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if workspace is None:
        need = _lib.decode_workspace_bytes(B, Hq, Hkv, D)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if stream is not None:
            workspace.record_stream(st)
    if isinstance(q_pos, torch.Tensor):
        if (q_pos.dtype != torch.int32 or q_pos.device != q.device or tuple(q_pos.shape) != (B,)
                or not q_pos.is_contiguous()):
            raise ValueError("q_pos must be an int32 GPU tensor of shape (B,) on q's device")
        bound = S_cap - 1 if max_pos is None else int(max_pos)
        rc = _lib.decode_ragged_raw(q.data_ptr(), cache.data_ptr(), cache.numel(), B, S_cap, Hq, Hkv, D, rope_theta,
                                    q_pos.data_ptr(), bound, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), st.cuda_stream, rope_style=_rope_style(interleaved))
        if rc != _lib.ATTN_OK:
            raise _lib.AttnError(rc, "attn_decode_ragged")
        return out, lse
    rc = _lib.decode_raw(q.data_ptr(), cache.data_ptr(), cache.numel(), B, S_cap, Hq, Hkv, D, rope_theta, q_pos,
                         out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), workspace.numel(), st.cuda_stream,
                         rope_style=_rope_style(interleaved))
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_decode")
    return out, lse


def attn_bwd(q, k, v, out, lse, dout, rope_theta, causal=True, dq=None, dk=None, dv=None, workspace=None,
             stream=None, interleaved=False, q_pos0=0, k_pos0=0):
    """Gradients (dq, dk, dv) of attn_fwd's out for the output gradient dout (bf16).

    out, lse: attn_fwd's results for the same q, k, v, rope_theta, causal and interleaved.
    With q_pos0 / k_pos0 the call is one step of ring attention's backward (attn_bwd_shard):
    out and lse must then be the merged forward results of these queries over every key block,
    and the returned gradients are this pair of blocks' parts (dq summed over key blocks, dk and
    dv over query blocks give the whole sequence's).
    """
    B, S, Hq, Hkv, D = _shapes(q, k, v)
    if q.dtype != torch.bfloat16:
        raise TypeError("attn_bwd takes bfloat16 tensors")
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor shaped and typed like q")
    if tuple(lse.shape) != (B, Hq, S) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, Hq, S)")
    made = (torch.empty_like(q) if dq is None else None, torch.empty_like(k) if dk is None else None,
            torch.empty_like(v) if dv is None else None)
    dq = made[0] if dq is None else dq
    dk = made[1] if dk is None else dk
    dv = made[2] if dv is None else dv
    _keep_for(stream, *made)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor shaped and typed like {name[1:]}")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    if workspace is None:
        workspace = torch.empty(_lib.bwd_workspace_bytes(B, S, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
        if stream is not None:
            workspace.record_stream(st)
    rc = _lib.bwd_shard_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), B, S, Hq, Hkv, D, rope_theta, 1 if causal else 0, q_pos0, k_pos0,
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                            st.cuda_stream, rope_style=_rope_style(interleaved))
    if rc != _lib.ATTN_OK:
        raise _lib.AttnError(rc, "attn_bwd_shard" if (q_pos0 or k_pos0) else "attn_bwd")
    return dq, dk, dv
