"""attn_fp4_fwd_kvcache_noalloc (the cache forward for callers that cannot allocate) against
attn_fp4_fwd_kvcache with a caller-given workspace, through the C ABI.

Both run the same kernels on the same split plan, so O, m and l must be bit-identical.  Two calls
in a row, the second with a smaller input, show that the library's scratch array is reused
correctly.  A shape whose split workspace exceeds the array is refused before any launch (that
check needs no GPU).
"""

import ctypes

import numpy as np
import pytest

from bit_attention_amd import ops
from bit_attention_amd import workloads as W


def _inputs(seed, B, Hq, Hkv, Nk, d):
    import torch
    r = np.random.default_rng(seed)
    q = W.round_to_bf16(r.standard_normal((B, Hq, 1, d)) * 1.5)
    k = W.round_to_bf16(r.standard_normal((B, Hkv, Nk, d)))
    v = W.round_to_bf16(r.standard_normal((B, Hkv, Nk, d)))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()  # noqa: E731
    return (*ops.attn_fp4_quantize(dev(q), 0), *ops.attn_fp4_quantize(dev(k), 0),
            *ops.attn_fp4_quantize(dev(v), 1))


@pytest.mark.gpu
def test_noalloc_matches_workspace_path_twice():
    import torch
    for seed, (B, Hq, Hkv, Nk, d), lens in ((11, (4, 16, 4, 8192, 128), [8192, 5000, 64, 7777]),
                                            (12, (2, 8, 2, 2048, 64), [2048, 1000])):
        assert ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, 1, Nk, d) > 0   # the split path
        args = _inputs(seed, B, Hq, Hkv, Nk, d)
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        o1, m1, l1 = ops.attn_fp4_fwd_kvcache(*args, seqlens_k=sl, causal=True)
        o2 = torch.full_like(o1, float("nan"))
        m2 = torch.full_like(m1, float("nan"))
        l2 = torch.full_like(l1, float("nan"))
        ops.attn_fp4_fwd_kvcache_noalloc(*args, seqlens_k=sl, causal=True, o=o2, m=m2, l=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(m1, m2) and torch.equal(l1, l2), (B, Hq, Hkv, Nk, d)
        assert torch.isfinite(o2).all()


def test_noalloc_refuses_a_split_workspace_above_its_array():
    # one KV head with 16320 new rows against a 65536-key cache: the split workspace is ~42 MB
    B, Hq, Hkv, Nq, Nk, d = 1, 1, 1, 16320, 65536, 128
    need = ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    assert need > ops.KVCACHE_SCRATCH_BYTES
    a = ops.FwdKvcacheArgs(*([16] * 6), None, 16, 16, 16, None, 0, B, Hq, Hkv, Nq, Nk, d, 1, 0.0, 0)
    st = ops.lib().attn_fp4_fwd_kvcache_noalloc(ctypes.byref(a), None)
    assert ops.STATUS[st] == "ATTN_FP4_E_WORKSPACE"
    # invalid sizes are refused as by attn_fp4_fwd_kvcache
    a.Nk = 100
    assert ops.STATUS[ops.lib().attn_fp4_fwd_kvcache_noalloc(ctypes.byref(a), None)] == "ATTN_FP4_E_INVALID_ARG"
