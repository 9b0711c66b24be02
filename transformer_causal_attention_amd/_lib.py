"""ctypes binding of libattn.so (the C ABI declared in include/attn.h).

Only argument marshalling lives here; every step of the computation runs in the HIP
kernels behind the C ABI.  Loading fails loudly when the library has not been built.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_DTYPE_BF16 = 0
ATTN_DTYPE_FP32 = 1

ATTN_ROPE_HALF = 0
ATTN_ROPE_INTERLEAVED = 1

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EHIP = -3
ATTN_EWORKSPACE = -4
ATTN_ESCRATCH = -5

# Every symbol include/attn.h declares, with its ctypes signature.
_VP = ctypes.c_void_p
_I = ctypes.c_int
_FWD_ARGS = [_VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_double, _I, _I, _I, _VP, _VP, _VP, ctypes.c_size_t, _VP]
_SHARD_ARGS = [_VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_double, _I, _I, _I, _I, _I, _VP, _VP, _VP, ctypes.c_size_t,
               _VP]
_MERGE_ARGS = [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _VP, _VP, _VP]
_PREP_ARGS = [_VP, _VP, _I, _I, _I, _I, ctypes.c_double, _I, _I, _I, _VP, ctypes.c_size_t, _VP]
_BWD_ARGS = [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_double, _I, _I, _VP, _VP, _VP, _VP,
             ctypes.c_size_t, _VP]
_DECODE_ARGS = [_VP, _VP, ctypes.c_size_t, _I, _I, _I, _I, _I, ctypes.c_double, _I, _I, _VP, _VP, _VP, ctypes.c_size_t,
                _VP]
SIGNATURES = {
    "attn_abi_version": (_I, []),
    "attn_strerror": (ctypes.c_char_p, [_I]),
    "attn_fwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "attn_fwd": (_I, _FWD_ARGS),
    "attn_fwd_timed": (_I, _FWD_ARGS + [_VP, _VP]),
    "attn_fwd_noalloc": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_double, _I, _I, _I, _VP, _VP, _VP]),
    "attn_fwd_shard": (_I, _SHARD_ARGS),
    "attn_merge": (_I, _MERGE_ARGS),
    "attn_kv_prepare": (_I, _PREP_ARGS),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_decode": (_I, _DECODE_ARGS),
    "attn_decode_ragged": (_I, _DECODE_ARGS[:10] + [_VP, _I] + _DECODE_ARGS[11:]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "attn_bwd": (_I, _BWD_ARGS),
    "attn_bwd_shard": (_I, _BWD_ARGS[:14] + [_I, _I] + _BWD_ARGS[14:]),
    "attn_event_create": (_VP, []),
    "attn_event_destroy": (_I, [_VP]),
    "attn_event_elapsed_ms": (_I, [_VP, _VP, ctypes.POINTER(ctypes.c_float)]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load():
    """Load libattn.so once and attach the C signatures.  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m transformer_causal_attention_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def strerror(code):
    return load().attn_strerror(int(code)).decode()


def abi_version():
    return load().attn_abi_version()


def workspace_bytes(B, S, Hkv, head_dim, dtype):
    return load().attn_fwd_workspace_bytes(B, S, Hkv, head_dim, dtype)


def fwd_raw(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, causal, dtype, out, lse, workspace,
            workspace_bytes_, stream, ev_start=None, ev_stop=None, rope_style=ATTN_ROPE_HALF):
    """Call attn_fwd (or attn_fwd_timed when events are given) with raw pointers; returns the code."""
    lib = load()
    args = (q, k, v, B, S, Hq, Hkv, head_dim, float(rope_theta), int(rope_style), int(causal), dtype, out, lse,
            workspace, workspace_bytes_, stream)
    if ev_start is None and ev_stop is None:
        return lib.attn_fwd(*args)
    return lib.attn_fwd_timed(*args, ev_start, ev_stop)


def fwd_noalloc_raw(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, causal, dtype, out, lse, stream,
                    rope_style=ATTN_ROPE_HALF):
    """Call attn_fwd_noalloc (the library's own scratch as workspace) with raw pointers; returns the code."""
    return load().attn_fwd_noalloc(q, k, v, B, S, Hq, Hkv, head_dim, float(rope_theta), int(rope_style), int(causal),
                                   dtype, out, lse, stream)


def shard_raw(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, causal, q_pos0, k_pos0, dtype, out, lse,
              workspace, workspace_bytes_, stream, rope_style=ATTN_ROPE_HALF):
    """Call attn_fwd_shard with raw pointers; returns the code."""
    return load().attn_fwd_shard(q, k, v, B, S, Hq, Hkv, head_dim, float(rope_theta), int(rope_style), int(causal),
                                 int(q_pos0), int(k_pos0), dtype, out, lse, workspace, workspace_bytes_, stream)


def merge_raw(o1, lse1, o2, lse2, B, S, H, head_dim, dtype, out, lse, stream):
    """Call attn_merge with raw pointers; returns the code."""
    return load().attn_merge(o1, lse1, o2, lse2, B, S, H, head_dim, dtype, out, lse, stream)


def kv_prepare_raw(k, v, B, S_cap, Hkv, head_dim, rope_theta, key0, key1, cache, cache_bytes, stream,
                   rope_style=ATTN_ROPE_HALF):
    """Call attn_kv_prepare with raw pointers; returns the code."""
    return load().attn_kv_prepare(k, v, B, S_cap, Hkv, head_dim, float(rope_theta), int(rope_style), int(key0),
                                  int(key1), cache, cache_bytes, stream)


def decode_workspace_bytes(B, Hq, Hkv, head_dim):
    return load().attn_decode_workspace_bytes(B, Hq, Hkv, head_dim)


def decode_raw(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, rope_theta, q_pos, out, lse, workspace,
               workspace_bytes_, stream, rope_style=ATTN_ROPE_HALF):
    """Call attn_decode with raw pointers; returns the code."""
    return load().attn_decode(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, float(rope_theta), int(rope_style),
                              int(q_pos), out, lse, workspace, workspace_bytes_, stream)


def decode_ragged_raw(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, rope_theta, q_pos, max_pos, out, lse,
                      workspace, workspace_bytes_, stream, rope_style=ATTN_ROPE_HALF):
    """Call attn_decode_ragged (q_pos: device pointer to B int32 positions); returns the code."""
    return load().attn_decode_ragged(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, float(rope_theta),
                                     int(rope_style), q_pos, int(max_pos), out, lse, workspace, workspace_bytes_,
                                     stream)


def bwd_workspace_bytes(B, S, Hq, Hkv, head_dim):
    return load().attn_bwd_workspace_bytes(B, S, Hq, Hkv, head_dim)


def bwd_raw(q, k, v, out, lse, dout, B, S, Hq, Hkv, head_dim, rope_theta, causal, dq, dk, dv, workspace,
            workspace_bytes_, stream, rope_style=ATTN_ROPE_HALF):
    """Call attn_bwd with raw pointers; returns the code."""
    return load().attn_bwd(q, k, v, out, lse, dout, B, S, Hq, Hkv, head_dim, float(rope_theta), int(rope_style),
                           int(causal), dq, dk, dv, workspace, workspace_bytes_, stream)


def bwd_shard_raw(q, k, v, out, lse, dout, B, S, Hq, Hkv, head_dim, rope_theta, causal, q_pos0, k_pos0, dq, dk, dv,
                  workspace, workspace_bytes_, stream, rope_style=ATTN_ROPE_HALF):
    """Call attn_bwd_shard with raw pointers; returns the code."""
    return load().attn_bwd_shard(q, k, v, out, lse, dout, B, S, Hq, Hkv, head_dim, float(rope_theta), int(rope_style),
                                 int(causal), int(q_pos0), int(k_pos0), dq, dk, dv, workspace, workspace_bytes_, stream)


class Event:
    """A HIP timing event owned by the library (attn_event_create / destroy)."""

    def __init__(self):
        self.ptr = load().attn_event_create()
        if not self.ptr:
            raise AttnError(ATTN_EHIP, "attn_event_create")

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.attn_event_destroy(self.ptr)
            self.ptr = None

    def elapsed_ms(self, stop):
        ms = ctypes.c_float()
        rc = load().attn_event_elapsed_ms(self.ptr, stop.ptr, ctypes.byref(ms))
        if rc != ATTN_OK:
            raise AttnError(rc, "attn_event_elapsed_ms")
        return ms.value
