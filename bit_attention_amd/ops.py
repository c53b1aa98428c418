"""Thin ctypes binding of libattnfp4.so (same entry-point names as include/attn_fp4.h).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
If the library is missing or fails to load, every call raises -- there is no
fallback path.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnfp4.so")

STATUS = {
    0: "ATTN_FP4_OK",
    1: "ATTN_FP4_E_INVALID_ARG",
    2: "ATTN_FP4_E_UNSUPPORTED_DEVICE",
    3: "ATTN_FP4_E_UNSUPPORTED",
    4: "ATTN_FP4_E_HIP",
    5: "ATTN_FP4_E_WORKSPACE",
}

EXPORTED = (
    "attn_fp4_abi_version",
    "attn_fp4_status_string",
    "attn_fp4_quantize",
    "attn_fp4_fwd",
    "attn_fp4_fwd_kvcache",
    "attn_fp4_fwd_kvcache_workspace_bytes",
    "attn_fp4_fwd_kvcache_noalloc",
    "attn_fp4_bwd_workspace_bytes",
    "attn_fp4_bwd_recompute",
    "attn_fp4_nv_quantize",
    "attn_fp4_nv_fwd_workspace_bytes",
    "attn_fp4_nv_fwd",
)


class AttnFp4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(status, status), _status_string(status)))


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("N", ctypes.c_int64), ("d", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("p_rule", ctypes.c_int32),
    ]


class NvFwdArgs(ctypes.Structure):
    _fields_ = [
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("q_tensor_scale", ctypes.c_void_p), ("k_tensor_scale", ctypes.c_void_p),
        ("v_tensor_scale", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("N", ctypes.c_int64), ("d", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


P_EXP, P_EFQ = 0, 1   # P~ rules of the forward (exp-then-quantize; exp-free EFQ codes)


class FwdKvcacheArgs(ctypes.Structure):
    _fields_ = [
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("seqlens_k", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("d", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("p_rule", ctypes.c_int32),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("do_", ctypes.c_void_p),
        ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("N", ctypes.c_int64), ("d", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


_lib = None


def lib():
    """Load libattnfp4.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libattnfp4.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.attn_fp4_abi_version.restype = ctypes.c_int32
        L.attn_fp4_status_string.restype = ctypes.c_char_p
        L.attn_fp4_status_string.argtypes = [ctypes.c_int32]
        L.attn_fp4_quantize.restype = ctypes.c_int32
        L.attn_fp4_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.attn_fp4_fwd.restype = ctypes.c_int32
        L.attn_fp4_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        L.attn_fp4_fwd_kvcache.restype = ctypes.c_int32
        L.attn_fp4_fwd_kvcache.argtypes = [ctypes.POINTER(FwdKvcacheArgs), ctypes.c_void_p]
        L.attn_fp4_fwd_kvcache_noalloc.restype = ctypes.c_int32
        L.attn_fp4_fwd_kvcache_noalloc.argtypes = [ctypes.POINTER(FwdKvcacheArgs), ctypes.c_void_p]
        L.attn_fp4_fwd_kvcache_workspace_bytes.restype = ctypes.c_int64
        L.attn_fp4_fwd_kvcache_workspace_bytes.argtypes = [ctypes.c_int64] * 6
        L.attn_fp4_bwd_workspace_bytes.restype = ctypes.c_int64
        L.attn_fp4_bwd_workspace_bytes.argtypes = [ctypes.c_int64] * 5
        L.attn_fp4_bwd_recompute.restype = ctypes.c_int32
        L.attn_fp4_bwd_recompute.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p]
        L.attn_fp4_nv_quantize.restype = ctypes.c_int32
        L.attn_fp4_nv_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]
        L.attn_fp4_nv_fwd_workspace_bytes.restype = ctypes.c_int64
        L.attn_fp4_nv_fwd_workspace_bytes.argtypes = [ctypes.c_int64] * 5
        L.attn_fp4_nv_fwd.restype = ctypes.c_int32
        L.attn_fp4_nv_fwd.argtypes = [ctypes.POINTER(NvFwdArgs), ctypes.c_void_p]
        _lib = L
    return _lib


def _status_string(status):
    try:
        return lib().attn_fp4_status_string(status).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(status, what):
    if status != 0:
        raise AttnFp4Error(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))


def attn_fp4_abi_version():
    return int(lib().attn_fp4_abi_version())


def attn_fp4_quantize(x, axis, codes=None, scales=None, stream=None):
    """MXFP4-quantize bf16 ``x`` [..., n, d].

    axis=0: along d -> codes [..., n, d/2], scales [..., n, d/32] (uint8).
    axis=1: along n, block-major -> codes [..., n/32, d, 16], scales [..., n/32, d]
            (for each 32-token block, the 16 code bytes of every channel).
    """
    _dev(x, torch.bfloat16, "x")
    *lead, n, d = x.shape
    bh = int(math.prod(lead)) if lead else 1
    if axis == 0:
        cshape, sshape = (*lead, n, d // 2), (*lead, n, d // 32)
    else:
        cshape, sshape = (*lead, n // 32, d, 16), (*lead, n // 32, d)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    _check(lib().attn_fp4_quantize(_ptr(x), bh, n, d, int(axis), _ptr(codes), _ptr(scales), _stream(stream)),
           "attn_fp4_quantize")
    return codes, scales


def attn_fp4_fwd(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, causal=False,
                 softmax_scale=0.0, o=None, m=None, l=None, stream=None, p_rule=P_EXP):
    """MXFP4 attention forward on pre-quantized operands (layouts of attn_fp4_quantize).

    q_codes [B, Hq, N, d/2]; k_codes [B, Hkv, N, d/2]; v_codes [B, Hkv, N/32, d, 16].
    Returns (o bf16 [B, Hq, N, d], m fp32 [B, Hq, N], l fp32 [B, Hq, N]).
    """
    B, Hq, N, dh = q_codes.shape
    d = 2 * dh
    Hkv = k_codes.shape[1]
    for t, name in ((q_codes, "q_codes"), (q_scales, "q_scales"), (k_codes, "k_codes"),
                    (k_scales, "k_scales"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, torch.uint8, name)
    if k_codes.shape != (B, Hkv, N, dh) or v_codes.shape != (B, Hkv, N // 32, d, 16):
        raise ValueError("inconsistent operand shapes")
    if q_scales.shape != (B, Hq, N, d // 32) or k_scales.shape != (B, Hkv, N, d // 32) \
            or v_scales.shape != (B, Hkv, N // 32, d):
        raise ValueError("inconsistent scale shapes")
    dev = q_codes.device
    if o is None:
        o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    if m is None:
        m = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    a = FwdArgs(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                _ptr(o), _ptr(m), _ptr(l), B, Hq, Hkv, N, d, int(bool(causal)), float(softmax_scale), int(p_rule))
    _check(lib().attn_fp4_fwd(ctypes.byref(a), _stream(stream)), "attn_fp4_fwd")
    return o, m, l


def attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d):
    return int(lib().attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def _kvcache_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, seqlens_k, causal, softmax_scale,
                  o, m, l, p_rule, workspace):
    """Check the cache forward's operands, allocate missing outputs, fill the argument struct.
    workspace: "auto", None or a uint8 CUDA tensor (see attn_fp4_fwd_kvcache)."""
    B, Hq, Nq, dh = q_codes.shape
    d = 2 * dh
    Hkv, Nk = k_codes.shape[1], k_codes.shape[2]
    for t, name in ((q_codes, "q_codes"), (q_scales, "q_scales"), (k_codes, "k_codes"),
                    (k_scales, "k_scales"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, torch.uint8, name)
    if k_codes.shape != (B, Hkv, Nk, dh) or v_codes.shape != (B, Hkv, Nk // 32, d, 16):
        raise ValueError("inconsistent operand shapes")
    if q_scales.shape != (B, Hq, Nq, d // 32) or k_scales.shape != (B, Hkv, Nk, d // 32) \
            or v_scales.shape != (B, Hkv, Nk // 32, d):
        raise ValueError("inconsistent scale shapes")
    if seqlens_k is not None:
        _dev(seqlens_k, torch.int32, "seqlens_k")
        if seqlens_k.shape != (B,):
            raise ValueError("seqlens_k must be [B]")
    dev = q_codes.device
    if o is None:
        o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    if m is None:
        m = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
    a = FwdKvcacheArgs(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                       _ptr(v_scales), None if seqlens_k is None else _ptr(seqlens_k),
                       _ptr(o), _ptr(m), _ptr(l),
                       None if workspace is None else _ptr(workspace),
                       0 if workspace is None else workspace.numel(),
                       B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(softmax_scale), int(p_rule))
    return a, o, m, l


def attn_fp4_fwd_kvcache(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, seqlens_k=None,
                         causal=False, softmax_scale=0.0, o=None, m=None, l=None, stream=None, p_rule=P_EXP,
                         workspace="auto"):
    """Forward of Nq new query rows against a pre-quantized key/value cache of capacity Nk.

    q_codes [B, Hq, Nq, d/2]; k_codes [B, Hkv, Nk, d/2]; v_codes [B, Hkv, Nk/32, d, 16] (the cache
    quantized as a whole); seqlens_k: int32 device tensor [B] of valid cache lengths, or None for
    Nk.  The new rows are the last Nq positions of each sequence (bottom-right causal alignment).
    workspace: "auto" allocates the split forward's workspace when the shape uses one; None runs
    the one-pass kernel; a uint8 CUDA tensor is used as given.
    Returns (o bf16 [B, Hq, Nq, d], m fp32 [B, Hq, Nq], l fp32 [B, Hq, Nq]).
    """
    a, o, m, l = _kvcache_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, seqlens_k, causal,
                               softmax_scale, o, m, l, p_rule, workspace)
    _check(lib().attn_fp4_fwd_kvcache(ctypes.byref(a), _stream(stream)), "attn_fp4_fwd_kvcache")
    return o, m, l


KVCACHE_SCRATCH_BYTES = 16 * 1024 * 1024   # ATTN_FP4_KVCACHE_SCRATCH_BYTES of include/attn_fp4.h


def attn_fp4_fwd_kvcache_noalloc(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, seqlens_k=None,
                                 causal=False, softmax_scale=0.0, o=None, m=None, l=None, stream=None,
                                 p_rule=P_EXP):
    """attn_fp4_fwd_kvcache whose split workspace is the library's own device array (the C call
    allocates nothing; pass o, m, l to allocate nothing here either).  Calls that overlap on one
    GPU share that array and race."""
    a, o, m, l = _kvcache_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, seqlens_k, causal,
                               softmax_scale, o, m, l, p_rule, None)
    _check(lib().attn_fp4_fwd_kvcache_noalloc(ctypes.byref(a), _stream(stream)), "attn_fp4_fwd_kvcache_noalloc")
    return o, m, l


def attn_fp4_bwd_workspace_bytes(B, Hq, Hkv, N, d):
    return int(lib().attn_fp4_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def attn_fp4_bwd_recompute(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, o, do, m, l,
                           causal=False, softmax_scale=0.0, dq=None, dk=None, dv=None, workspace=None,
                           stream=None):
    """Attn-QAT backward: returns (dq, dk, dv) bf16."""
    B, Hq, N, dh = q_codes.shape
    d = 2 * dh
    Hkv = k_codes.shape[1]
    dev = q_codes.device
    if k_codes.shape != (B, Hkv, N, dh) or v_codes.shape != (B, Hkv, N // 32, d, 16) \
            or v_scales.shape != (B, Hkv, N // 32, d):
        raise ValueError("inconsistent operand shapes")
    _dev(o, torch.bfloat16, "o")
    _dev(do, torch.bfloat16, "do")
    _dev(m, torch.float32, "m")
    _dev(l, torch.float32, "l")
    if dq is None:
        dq = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    if dk is None:
        dk = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    need = attn_fp4_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if need < 0:
        raise AttnFp4Error(1, "attn_fp4_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    a = BwdArgs(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                _ptr(o), _ptr(do), _ptr(m), _ptr(l), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                workspace.numel(), B, Hq, Hkv, N, d, int(bool(causal)), float(softmax_scale))
    _check(lib().attn_fp4_bwd_recompute(ctypes.byref(a), _stream(stream)), "attn_fp4_bwd_recompute")
    return dq, dk, dv


def attn_fp4_nv_quantize(x, axis, codes=None, scales=None, tensor_scale=None, stream=None):
    """NVFP4-style quantization of bf16 ``x`` [..., n, d] (16-element blocks, E4M3 scales).

    axis=0: along d -> codes [..., n, d/2], scales [..., n, d/16].
    axis=1: along n, transposed -> codes [..., d, n/2], scales [..., d, n/16].
    tensor_scale: float32 [2] on the device, written with (G, amax).
    Returns (codes, scales, tensor_scale).
    """
    _dev(x, torch.bfloat16, "x")
    *lead, n, d = x.shape
    bh = int(math.prod(lead)) if lead else 1
    if axis == 0:
        cshape, sshape = (*lead, n, d // 2), (*lead, n, d // 16)
    else:
        cshape, sshape = (*lead, d, n // 2), (*lead, d, n // 16)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    if tensor_scale is None:
        tensor_scale = torch.empty(2, dtype=torch.float32, device=x.device)
    _check(lib().attn_fp4_nv_quantize(_ptr(x), bh, n, d, int(axis), _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                                      _stream(stream)), "attn_fp4_nv_quantize")
    return codes, scales, tensor_scale


def attn_fp4_nv_fwd_workspace_bytes(B, Hq, Hkv, N, d):
    return int(lib().attn_fp4_nv_fwd_workspace_bytes(B, Hq, Hkv, N, d))


def attn_fp4_nv_fwd(q_codes, q_scales, q_ts, k_codes, k_scales, k_ts, v_codes, v_scales, v_ts, causal=False,
                    softmax_scale=0.0, o=None, m=None, l=None, workspace=None, stream=None):
    """Attention forward on NVFP4-style operands (layouts and tensor scales of attn_fp4_nv_quantize).

    q_codes [B, Hq, N, d/2]; k_codes [B, Hkv, N, d/2]; v_codes [B, Hkv, d, N/2]; *_ts float32 [2].
    Returns (o bf16 [B, Hq, N, d], m fp32 [B, Hq, N], l fp32 [B, Hq, N]).
    """
    B, Hq, N, dh = q_codes.shape
    d = 2 * dh
    Hkv = k_codes.shape[1]
    for t, name in ((q_codes, "q_codes"), (q_scales, "q_scales"), (k_codes, "k_codes"),
                    (k_scales, "k_scales"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, torch.uint8, name)
    for t, name in ((q_ts, "q_ts"), (k_ts, "k_ts"), (v_ts, "v_ts")):
        _dev(t, torch.float32, name)
    if k_codes.shape != (B, Hkv, N, dh) or v_codes.shape != (B, Hkv, d, N // 2):
        raise ValueError("inconsistent operand shapes")
    if q_scales.shape != (B, Hq, N, d // 16) or k_scales.shape != (B, Hkv, N, d // 16) \
            or v_scales.shape != (B, Hkv, d, N // 16):
        raise ValueError("inconsistent scale shapes")
    dev = q_codes.device
    if o is None:
        o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    if m is None:
        m = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    if l is None:
        l = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    need = attn_fp4_nv_fwd_workspace_bytes(B, Hq, Hkv, N, d)
    if need < 0:
        raise AttnFp4Error(1, "attn_fp4_nv_fwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    a = NvFwdArgs(_ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                  _ptr(q_ts), _ptr(k_ts), _ptr(v_ts), _ptr(o), _ptr(m), _ptr(l), _ptr(workspace), workspace.numel(),
                  B, Hq, Hkv, N, d, int(bool(causal)), float(softmax_scale))
    _check(lib().attn_fp4_nv_fwd(ctypes.byref(a), _stream(stream)), "attn_fp4_nv_fwd")
    return o, m, l
