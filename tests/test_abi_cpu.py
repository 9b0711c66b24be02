"""The C ABI library on a machine without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented codes before any HIP call."""

import ctypes
import os
import re

import pytest

from transformer_causal_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libattn.so not built")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_strerror", "attn_abi_version", "attn_fwd_workspace_bytes"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def declared_arity():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(attn_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_the_header():
    arity = declared_arity()
    assert set(arity) == set(_lib.SIGNATURES)
    for name, (_, args) in _lib.SIGNATURES.items():
        assert len(args) == arity[name], f"{name}: binding has {len(args)} arguments, header {arity[name]}"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_version_and_strerror():
    assert _lib.abi_version() == 6
    for code in (0, -1, -2, -3, -4, -5):
        assert len(_lib.strerror(code)) > 5
    assert "unknown" in _lib.strerror(12345)


def _flag_area(B, S, Hkv):
    # one 8-byte tag per tile half, then a 4-byte status word, padded to 256 bytes
    n = B * Hkv * ((S + 63) // 64) * 2
    return (n * 8 + 16 + 255) // 256 * 256


def test_workspace_bytes():
    # bf16: rotated keys and transposed values, each (B, Hkv, S rounded up to 64, D) bf16, then
    # the one-launch form's flag area (not at head_dim 256, which has no such form)
    assert _lib.workspace_bytes(1, 2048, 8, 128, 0) == 2 * 1 * 8 * 2048 * 128 * 2 + _flag_area(1, 2048, 8)
    assert _lib.workspace_bytes(2, 100, 3, 64, 0) == 2 * 2 * 3 * 128 * 64 * 2 + _flag_area(2, 100, 3)
    assert _lib.workspace_bytes(1, 1, 1, 64, 0) == 2 * 64 * 64 * 2 + _flag_area(1, 1, 1)
    assert _lib.workspace_bytes(1, 64, 1, 64, 1) == 0  # fp32 needs none
    assert _lib.workspace_bytes(1, 64, 1, 96, 0) == 0  # unsupported -> 0
    assert _lib.workspace_bytes(1, 100, 1, 256, 0) == 2 * 128 * 256 * 2  # head_dim 256 (bf16 forward)
    assert _lib.workspace_bytes(0, 64, 1, 64, 0) == 0


# Fake, aligned, non-null "device pointers": every call below must be rejected on the host
# before any HIP call, so they are never dereferenced.
P = 0x10000


def call(**over):
    a = dict(q=P, k=P, v=P, B=1, S=64, Hq=4, Hkv=1, d=64, theta=10000.0, causal=1, dtype=0,
             out=P, lse=P, ws=P, wsb=1 << 30, stream=None, rope=0)
    a.update(over)
    return _lib.fwd_raw(a["q"], a["k"], a["v"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["theta"],
                        a["causal"], a["dtype"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"],
                        rope_style=a["rope"])


@pytest.mark.parametrize("over", [
    dict(q=None), dict(k=None), dict(v=None), dict(out=None), dict(lse=None),
    dict(q=P + 8), dict(k=P + 2), dict(v=P + 4), dict(out=P + 1), dict(lse=P + 2),
    dict(B=0), dict(S=0), dict(Hq=0), dict(Hkv=0), dict(B=-3), dict(S=-1),
    dict(Hq=6, Hkv=4), dict(Hq=3, Hkv=2),
    dict(theta=0.0), dict(theta=-1.0), dict(theta=float("nan")), dict(theta=float("inf")),
    dict(causal=2), dict(causal=-1), dict(rope=2), dict(rope=-1),
])
def test_invalid_arguments(over):
    assert call(**over) == _lib.ATTN_EINVAL


@pytest.mark.parametrize("over", [
    dict(d=96), dict(d=512), dict(d=256, dtype=1), dict(d=32), dict(d=0), dict(dtype=2), dict(dtype=-1),
    dict(S=(1 << 28) + 1), dict(d=256, S=(1 << 22) + 1), dict(d=128, S=(1 << 23) - 63), dict(d=64, S=(1 << 24) - 63),
])
def test_unsupported(over):
    assert call(**over) == _lib.ATTN_EUNSUPPORTED


@pytest.mark.parametrize("over", [dict(ws=None), dict(wsb=1024), dict(ws=P + 8),
                                  dict(d=128, S=(1 << 23) - 64)])  # (the longest run 32-bit offsets allow)
def test_workspace_rejected(over):
    assert call(**over) == _lib.ATTN_EWORKSPACE


def test_timed_variant_validates_too():
    lib = _lib.load()
    rc = lib.attn_fwd_timed(P, P, P, 1, 64, 4, 1, 96, 1e4, 0, 1, 0, P, P, P, 1 << 30, None, None, None)
    assert rc == _lib.ATTN_EUNSUPPORTED
    rc = lib.attn_fwd_timed(P, P, P, 1, 64, 4, 1, 64, 1e4, 7, 1, 0, P, P, P, 1 << 30, None, None, None)
    assert rc == _lib.ATTN_EINVAL


def test_event_helpers_reject_null():
    lib = _lib.load()
    assert lib.attn_event_destroy(None) == _lib.ATTN_EINVAL
    ms = ctypes.c_float()
    assert lib.attn_event_elapsed_ms(None, None, ctypes.byref(ms)) == _lib.ATTN_EINVAL


def shard_call(**over):
    a = dict(q=P, k=P, v=P, B=1, S=64, Hq=4, Hkv=1, d=64, theta=10000.0, causal=1, qp=0, kp=0, dtype=0,
             out=P, lse=P, ws=P, wsb=1 << 30, stream=None, rope=0)
    a.update(over)
    return _lib.shard_raw(a["q"], a["k"], a["v"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["theta"],
                          a["causal"], a["qp"], a["kp"], a["dtype"], a["out"], a["lse"], a["ws"], a["wsb"],
                          a["stream"], rope_style=a["rope"])


@pytest.mark.parametrize("over", [
    dict(qp=-1), dict(kp=-5), dict(qp=(1 << 30) - 63), dict(kp=1 << 30), dict(q=None), dict(lse=P + 1),
    dict(Hq=3, Hkv=2), dict(causal=3), dict(rope=5),
])
def test_shard_invalid_arguments(over):
    assert shard_call(**over) == _lib.ATTN_EINVAL


@pytest.mark.parametrize("over,code", [
    (dict(d=96), _lib.ATTN_EUNSUPPORTED), (dict(dtype=5), _lib.ATTN_EUNSUPPORTED),
    (dict(wsb=16), _lib.ATTN_EWORKSPACE), (dict(ws=None), _lib.ATTN_EWORKSPACE),
])
def test_shard_other_rejections(over, code):
    assert shard_call(**over) == code


def merge_call(**over):
    a = dict(o1=P, l1=P, o2=P, l2=P, B=1, S=64, H=4, d=128, dtype=0, out=P, lse=P, stream=None)
    a.update(over)
    return _lib.merge_raw(a["o1"], a["l1"], a["o2"], a["l2"], a["B"], a["S"], a["H"], a["d"], a["dtype"],
                          a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("over", [
    dict(o1=None), dict(l1=None), dict(o2=None), dict(l2=None), dict(out=None), dict(lse=None),
    dict(o1=P + 8), dict(o2=P + 4), dict(out=P + 2), dict(l1=P + 1), dict(l2=P + 2), dict(lse=P + 3),
    dict(B=0), dict(S=0), dict(H=0), dict(S=-2),
])
def test_merge_invalid_arguments(over):
    assert merge_call(**over) == _lib.ATTN_EINVAL


@pytest.mark.parametrize("over", [dict(d=96), dict(d=512), dict(dtype=2), dict(dtype=-1)])
def test_merge_unsupported(over):
    assert merge_call(**over) == _lib.ATTN_EUNSUPPORTED


def test_decode_workspace_bytes():
    # partial (o, m, l) float32 rows: B * Hq heads * splits, with
    # splits = min(64, ceil(1024 / (B * Hkv * ceil(G / 32)))) at most
    assert _lib.decode_workspace_bytes(1, 32, 8, 128) == 32 * 64 * 130 * 4
    assert _lib.decode_workspace_bytes(8, 8, 1, 64) == 64 * 64 * 66 * 4
    assert _lib.decode_workspace_bytes(4, 32, 8, 128) == 128 * 32 * 130 * 4  # below the cap
    assert _lib.decode_workspace_bytes(2, 128, 2, 64) == 256 * 64 * 66 * 4  # 2 head blocks: 8 units
    assert _lib.decode_workspace_bytes(2048, 8, 1, 64) == 2048 * 8 * 66 * 4  # one split
    # head_dim 256: two-wave workgroups, so half as many splits (512 workgroups)
    assert _lib.decode_workspace_bytes(1, 48, 1, 256) == 48 * 64 * 258 * 4  # capped at 64
    assert _lib.decode_workspace_bytes(16, 48, 1, 256) == 16 * 48 * 16 * 258 * 4
    assert _lib.decode_workspace_bytes(4, 16, 16, 128) == 64 * 16 * 130 * 4
    assert _lib.decode_workspace_bytes(4, 16, 16, 256) == 64 * 8 * 258 * 4
    assert _lib.decode_workspace_bytes(1, 32, 8, 96) == 0
    assert _lib.decode_workspace_bytes(1, 6, 4, 64) == 0
    assert _lib.decode_workspace_bytes(0, 8, 1, 64) == 0


def prep_call(**over):
    a = dict(k=P, v=P, B=1, S=256, Hkv=2, d=64, theta=1e4, key0=0, key1=256, cache=P, cb=1 << 30, stream=None,
             rope=0)
    a.update(over)
    return _lib.kv_prepare_raw(a["k"], a["v"], a["B"], a["S"], a["Hkv"], a["d"], a["theta"], a["key0"], a["key1"],
                               a["cache"], a["cb"], a["stream"], rope_style=a["rope"])


@pytest.mark.parametrize("over,code", [
    (dict(k=None), _lib.ATTN_EINVAL), (dict(v=P + 8), _lib.ATTN_EINVAL), (dict(cache=None), _lib.ATTN_EINVAL),
    (dict(B=0), _lib.ATTN_EINVAL), (dict(S=0), _lib.ATTN_EINVAL), (dict(Hkv=-1), _lib.ATTN_EINVAL),
    (dict(theta=0.0), _lib.ATTN_EINVAL), (dict(theta=float("nan")), _lib.ATTN_EINVAL),
    (dict(key0=-1), _lib.ATTN_EINVAL), (dict(key0=5, key1=5), _lib.ATTN_EINVAL),
    (dict(key1=257), _lib.ATTN_EINVAL), (dict(key0=300, key1=301), _lib.ATTN_EINVAL),
    (dict(d=96), _lib.ATTN_EUNSUPPORTED), (dict(S=(1 << 28) + 1, key1=1), _lib.ATTN_EUNSUPPORTED),
    (dict(d=512), _lib.ATTN_EUNSUPPORTED), (dict(d=256, S=(1 << 22) + 1, key1=1), _lib.ATTN_EUNSUPPORTED),
    (dict(cb=2 * 2 * 256 * 64 * 2 - 1), _lib.ATTN_EWORKSPACE), (dict(rope=3), _lib.ATTN_EINVAL),
])
def test_kv_prepare_rejections(over, code):
    assert prep_call(**over) == code


def decode_call(**over):
    a = dict(q=P, cache=P, cb=1 << 30, B=1, S=256, Hq=8, Hkv=2, d=128, theta=1e4, pos=100, out=P, lse=P, ws=P,
             wsb=1 << 30, stream=None, rope=0)
    a.update(over)
    return _lib.decode_raw(a["q"], a["cache"], a["cb"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["theta"],
                           a["pos"], a["out"], a["lse"], a["ws"], a["wsb"], a["stream"], rope_style=a["rope"])


def test_decode_rejects_a_cache_smaller_than_its_layout():
    # the cache must hold the whole layout of (B, S_cap, Hkv, d): a larger S_cap, B or Hkv than
    # the allocation was made for is refused before any HIP call
    need = _lib.workspace_bytes(1, 256, 2, 128, 0)
    assert decode_call(cb=need - 1) == _lib.ATTN_EWORKSPACE
    assert decode_call(cb=need, S=512, pos=100) == _lib.ATTN_EWORKSPACE
    assert decode_call(cb=need, B=2) == _lib.ATTN_EWORKSPACE
    assert decode_call(cb=need, Hq=16, Hkv=4) == _lib.ATTN_EWORKSPACE
    assert decode_call(cb=0) == _lib.ATTN_EWORKSPACE


def test_unsupported_message_names_every_head_dim_rule():
    msg = _lib.strerror(_lib.ATTN_EUNSUPPORTED)
    assert "64 or 128" in msg and "256" in msg and "float32" in msg


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.ATTN_EINVAL), (dict(cache=P + 4), _lib.ATTN_EINVAL), (dict(out=P + 2), _lib.ATTN_EINVAL),
    (dict(lse=P + 1), _lib.ATTN_EINVAL), (dict(lse=None), _lib.ATTN_EINVAL),
    (dict(Hq=6, Hkv=4), _lib.ATTN_EINVAL), (dict(B=0), _lib.ATTN_EINVAL), (dict(theta=-2.0), _lib.ATTN_EINVAL),
    (dict(pos=-1), _lib.ATTN_EINVAL), (dict(pos=256), _lib.ATTN_EINVAL), (dict(rope=-1), _lib.ATTN_EINVAL),
    (dict(d=32), _lib.ATTN_EUNSUPPORTED), (dict(d=512), _lib.ATTN_EUNSUPPORTED),
    (dict(d=256, wsb=64), _lib.ATTN_EWORKSPACE),
    (dict(ws=None), _lib.ATTN_EWORKSPACE), (dict(wsb=64), _lib.ATTN_EWORKSPACE), (dict(ws=P + 4), _lib.ATTN_EWORKSPACE),
])
def test_decode_rejections(over, code):
    assert decode_call(**over) == code


def bwd_ws_expected(B, S, Hq, Hkv, d):
    # 3 key-side and 4 query-side tiles of 32 rows x d bf16 per block, 2 floats per query row,
    # and with HS > 1 head splits 2 x HS fp32 partial dk/dv blocks per K/V head.  HS: head_dim
    # 64/128 aim at 2048 waves of one key block each (key blocks in groups of 4), at most one
    # split per query head of the group; head_dim 256 at 512 workgroups of a key-block pair,
    # at most one split per pass of 4 heads.
    nb = (S + 31) // 32
    G = Hq // Hkv
    if d == 256:
        groups = B * Hkv * ((nb + 1) // 2)
        hs = max(1, min(-(-G // min(G, 4)), -(-512 // groups)))
    else:
        waves = B * Hkv * -(-nb // 4) * 4
        hs = max(1, min(G, -(-2048 // waves)))
    part = 2 * hs * B * Hkv * nb * 32 * d * 4 if hs > 1 else 0
    return (3 * B * Hkv + 4 * B * Hq) * nb * 32 * d * 2 + 2 * B * Hq * nb * 32 * 4 + part


def test_bwd_workspace_bytes():
    # B2 S100 Hq8 Hkv2 d128: 4 blocks, 16 waves -> 4 head splits (one per query head)
    nb = (100 + 31) // 32
    assert _lib.bwd_workspace_bytes(2, 100, 8, 2, 128) == ((3 * 2 * 2 + 4 * 2 * 8) * nb * 32 * 128 * 2
                                                           + 2 * 2 * 8 * nb * 32 * 4 + 2 * 4 * 2 * 2 * nb * 32 * 128 * 4)
    # Llama-3-8B backward: 64 blocks, 512 waves -> 4 splits; SmolLM MHA: one head per group
    for shape in [(2, 100, 8, 2, 128), (1, 2048, 32, 8, 128), (4, 1024, 32, 32, 64), (8, 1024, 8, 1, 64),
                  (1, 32768, 32, 8, 128), (1, 2048, 48, 1, 256), (1, 64, 4, 1, 64), (1, 64, 4, 1, 256)]:
        assert _lib.bwd_workspace_bytes(*shape) == bwd_ws_expected(*shape), shape
    assert _lib.bwd_workspace_bytes(1, 64, 4, 1, 96) == 0
    assert _lib.bwd_workspace_bytes(1, 64, 6, 4, 64) == 0


def bwd_call(**over):
    a = dict(q=P, k=P, v=P, out=P, lse=P, dout=P, B=1, S=64, Hq=4, Hkv=1, d=64, theta=1e4, causal=1, dq=P, dk=P,
             dv=P, ws=P, wsb=1 << 30, stream=None, rope=0)
    a.update(over)
    return _lib.bwd_raw(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["B"], a["S"], a["Hq"], a["Hkv"],
                        a["d"], a["theta"], a["causal"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], a["stream"],
                        rope_style=a["rope"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), _lib.ATTN_EINVAL), (dict(out=None), _lib.ATTN_EINVAL), (dict(lse=None), _lib.ATTN_EINVAL),
    (dict(dout=None), _lib.ATTN_EINVAL), (dict(dq=None), _lib.ATTN_EINVAL), (dict(dv=None), _lib.ATTN_EINVAL),
    (dict(k=P + 8), _lib.ATTN_EINVAL), (dict(dout=P + 2), _lib.ATTN_EINVAL), (dict(dk=P + 4), _lib.ATTN_EINVAL),
    (dict(lse=P + 2), _lib.ATTN_EINVAL), (dict(B=0), _lib.ATTN_EINVAL), (dict(S=-4), _lib.ATTN_EINVAL),
    (dict(Hq=3, Hkv=2), _lib.ATTN_EINVAL), (dict(causal=2), _lib.ATTN_EINVAL), (dict(theta=float("inf")), _lib.ATTN_EINVAL),
    (dict(rope=2), _lib.ATTN_EINVAL),
    (dict(d=96), _lib.ATTN_EUNSUPPORTED), (dict(S=(1 << 28) + 1), _lib.ATTN_EUNSUPPORTED),
    (dict(d=512), _lib.ATTN_EUNSUPPORTED), (dict(d=256, wsb=100), _lib.ATTN_EWORKSPACE),
    (dict(ws=None), _lib.ATTN_EWORKSPACE), (dict(wsb=100), _lib.ATTN_EWORKSPACE), (dict(ws=P + 8), _lib.ATTN_EWORKSPACE),
])
def test_bwd_rejections(over, code):
    assert bwd_call(**over) == code


def test_noalloc_rejections_before_any_hip_call():
    lib = _lib.load()
    # 2 * 8 * 2^20 * 128 * 2 bytes of tiles > the fixed scratch
    rc = lib.attn_fwd_noalloc(P, P, P, 1, 1 << 20, 32, 8, 128, 5e5, 0, 1, 0, P, P, None)
    assert rc == _lib.ATTN_ESCRATCH
    assert lib.attn_fwd_noalloc(None, P, P, 1, 64, 4, 1, 64, 1e4, 0, 1, 0, P, P, None) == _lib.ATTN_EINVAL
    assert lib.attn_fwd_noalloc(P, P, P, 1, 64, 4, 1, 96, 1e4, 0, 1, 0, P, P, None) == _lib.ATTN_EUNSUPPORTED
    assert "scratch" in _lib.strerror(_lib.ATTN_ESCRATCH)


def test_decode_ragged_rejections_before_any_hip_call():
    lib = _lib.load()
    args = lambda **o: dict(dict(q=P, cache=P, cb=1 << 30, B=2, S=256, Hq=8, Hkv=2, d=128, th=1e4, rope=0, qp=P,  # noqa: E731
                                 mp=100, out=P, lse=P, ws=P, wsb=1 << 30, st=None), **o)
    call_r = lambda a: _lib.decode_ragged_raw(a["q"], a["cache"], a["cb"], a["B"], a["S"], a["Hq"], a["Hkv"],  # noqa: E731
                                              a["d"], a["th"], a["qp"], a["mp"], a["out"], a["lse"], a["ws"],
                                              a["wsb"], a["st"], rope_style=a["rope"])
    assert call_r(args(qp=None)) == _lib.ATTN_EINVAL
    assert call_r(args(qp=P + 2)) == _lib.ATTN_EINVAL
    assert call_r(args(mp=256)) == _lib.ATTN_EINVAL  # max_pos must be below S_cap
    assert call_r(args(mp=-1)) == _lib.ATTN_EINVAL
    assert call_r(args(cb=16)) == _lib.ATTN_EWORKSPACE
    assert call_r(args(d=96)) == _lib.ATTN_EUNSUPPORTED
    assert lib is not None
