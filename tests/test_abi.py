"""The C-ABI library loads and exports every symbol include/attn_fp4.h declares (CPU only).

Only host-side argument validation is exercised here: every call below is rejected before
anything touches a device.
"""

import ctypes
import os
import re

import pytest

from bit_attention_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(attn_fp4_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(ops.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert ops.attn_fp4_abi_version() == 7


def test_status_strings():
    L = ops.lib()
    for s in range(6):
        assert L.attn_fp4_status_string(s)
    assert L.attn_fp4_status_string(99) == b"unknown status"


def test_host_validation_rejects_before_launch():
    L = ops.lib()
    # null / misaligned pointers and bad sizes are rejected on the host
    assert L.attn_fp4_quantize(None, 1, 32, 32, 0, None, None, None) == 1
    assert L.attn_fp4_quantize(ctypes.c_void_p(16), 1, 32, 33, 0, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 1
    assert L.attn_fp4_quantize(ctypes.c_void_p(16), 1, 32, 32, 2, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 1
    assert L.attn_fp4_quantize(ctypes.c_void_p(8), 1, 32, 32, 0, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 1
    a = ops.FwdArgs()
    assert L.attn_fp4_fwd(None, None) == 1
    assert L.attn_fp4_fwd(ctypes.byref(a), None) == 1          # zero dims
    p = ctypes.c_void_p(256)
    for kw in ({"N": 96}, {"d": 96}, {"Hkv": 3}):
        dims = dict(B=1, Hq=4, Hkv=2, N=128, d=128)
        dims.update(kw)
        a = ops.FwdArgs(p, p, p, p, p, p, p, p, p, dims["B"], dims["Hq"], dims["Hkv"], dims["N"], dims["d"], 0, 0.0)
        assert L.attn_fp4_fwd(ctypes.byref(a), None) == 1, kw
    # cache forward: capacity not a multiple of 64, Nq = 0, bad group, bad d, misaligned lengths
    assert L.attn_fp4_fwd_kvcache(None, None) == 1
    for kw in ({"Nk": 96}, {"Nq": 0}, {"Hkv": 3}, {"d": 96}, {"seq": ctypes.c_void_p(258)}, {"p_rule": 2}):
        dims = dict(B=1, Hq=4, Hkv=2, Nq=1, Nk=128, d=128, seq=None, p_rule=0)
        dims.update(kw)
        a = ops.FwdKvcacheArgs(p, p, p, p, p, p, dims["seq"], p, p, p, None, 0, dims["B"], dims["Hq"],
                               dims["Hkv"], dims["Nq"], dims["Nk"], dims["d"], 0, 0.0, dims["p_rule"])
        assert L.attn_fp4_fwd_kvcache(ctypes.byref(a), None) == 1, kw
    # split workspace: none needed for many rows; for decode-like shapes a positive size; a given
    # workspace that is too small is rejected
    assert L.attn_fp4_fwd_kvcache_workspace_bytes(1, 32, 8, 2048, 32768, 128) == 0
    need = L.attn_fp4_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 128)
    assert need > 0 and need % 256 == 0
    assert L.attn_fp4_fwd_kvcache_workspace_bytes(1, 4, 3, 1, 128, 128) == -1
    a = ops.FwdKvcacheArgs(p, p, p, p, p, p, None, p, p, p, ctypes.c_void_p(1 << 20), need - 256,
                           8, 32, 8, 1, 32768, 128, 0, 0.0, 0)
    assert L.attn_fp4_fwd_kvcache(ctypes.byref(a), None) == 5
    # one head's codes beyond the kernels' 32-bit buffer offsets: unsupported, before any launch
    big = 1 << 26
    a = ops.FwdArgs(p, p, p, p, p, p, p, p, p, 1, 1, 1, big, 128, 0, 0.0, 0)
    assert L.attn_fp4_fwd(ctypes.byref(a), None) == 3
    a = ops.FwdKvcacheArgs(p, p, p, p, p, p, None, p, p, p, None, 0, 1, 1, 1, 1, big, 128, 0, 0.0, 0)
    assert L.attn_fp4_fwd_kvcache(ctypes.byref(a), None) == 3
    # rows: 3 x [B*Hq*N] fp32; bf16 copies: V^ and K^T per KV head, Q^T and dO^T per query head
    assert L.attn_fp4_bwd_workspace_bytes(1, 2, 2, 128, 128) == 2 * 128 * 16 + 4 * (2 * 128 * 128 * 2)
    assert L.attn_fp4_bwd_workspace_bytes(1, 2, 2, 100, 128) < 0
    b = ops.BwdArgs(p, p, p, p, p, p, p, p, p, p, p, p, p, None, 0, 1, 2, 2, 128, 128, 0, 0.0)
    assert L.attn_fp4_bwd_recompute(ctypes.byref(b), None) == 5   # workspace missing
    # a KV head's group of bf16 [N, d] tensors beyond 2^31 bytes: unsupported (32-bit offsets)
    B, Hq, Hkv, N, d = 1, 64, 1, 1 << 18, 128
    need = L.attn_fp4_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    b = ops.BwdArgs(p, p, p, p, p, p, p, p, p, p, p, p, p, ctypes.c_void_p(1 << 20), need, B, Hq, Hkv, N, d, 0, 0.0)
    assert L.attn_fp4_bwd_recompute(ctypes.byref(b), None) == 3


def test_nv_host_validation_rejects_before_launch():
    L = ops.lib()
    p = ctypes.c_void_p(256)
    ts = ctypes.c_void_p(512)
    # tensor scale missing or misaligned, d not a multiple of 32, axis 1 with n % 16, bad axis
    assert L.attn_fp4_nv_quantize(p, 1, 32, 32, 0, p, p, None, None) == 1
    assert L.attn_fp4_nv_quantize(p, 1, 32, 32, 0, p, p, ctypes.c_void_p(516), None) == 1
    assert L.attn_fp4_nv_quantize(p, 1, 32, 48, 0, p, p, ts, None) == 1
    assert L.attn_fp4_nv_quantize(p, 1, 40, 32, 1, p, p, ts, None) == 1
    assert L.attn_fp4_nv_quantize(p, 1, 32, 32, 2, p, p, ts, None) == 1
    assert L.attn_fp4_nv_quantize(ctypes.c_void_p(8), 1, 32, 32, 0, p, p, ts, None) == 1
    # workspace: fp16 Q^ per query head, K^ and V^T per KV head, each region 256-aligned
    assert L.attn_fp4_nv_fwd_workspace_bytes(1, 4, 2, 128, 64) == 4 * 128 * 64 * 2 + 2 * (2 * 128 * 64 * 2)
    assert L.attn_fp4_nv_fwd_workspace_bytes(1, 4, 3, 128, 64) < 0
    assert L.attn_fp4_nv_fwd(None, None) == 1
    need = L.attn_fp4_nv_fwd_workspace_bytes(1, 4, 2, 128, 128)
    ws = ctypes.c_void_p(1 << 20)

    def args(**kw):
        a = dict(ts=ts, ws=ws, wsb=need, B=1, Hq=4, Hkv=2, N=128, d=128)
        a.update(kw)
        return ops.NvFwdArgs(p, p, p, p, p, p, a["ts"], a["ts"], a["ts"], p, p, p, a["ws"], a["wsb"],
                             a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], 0, 0.0)
    for kw in ({"N": 96}, {"d": 96}, {"Hkv": 3}, {"ts": None}, {"ts": ctypes.c_void_p(516)}):
        assert L.attn_fp4_nv_fwd(ctypes.byref(args(**kw)), None) == 1, kw
    assert L.attn_fp4_nv_fwd(ctypes.byref(args(ws=None)), None) == 5
    assert L.attn_fp4_nv_fwd(ctypes.byref(args(wsb=need - 256)), None) == 5
    assert L.attn_fp4_nv_fwd(ctypes.byref(args(ws=ctypes.c_void_p((1 << 20) + 16))), None) == 5
    # one head's bf16 operand beyond 2^31 bytes: unsupported (32-bit buffer offsets)
    big = 1 << 23
    a = args(N=big, Hq=1, Hkv=1, wsb=L.attn_fp4_nv_fwd_workspace_bytes(1, 1, 1, big, 128))
    assert L.attn_fp4_nv_fwd(ctypes.byref(a), None) == 3


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", "/nonexistent/libattnfp4.so")
    with pytest.raises(RuntimeError):
        ops.lib()
