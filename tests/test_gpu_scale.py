"""A caller-given softmax_scale (instead of 1/sqrt(d)) through every entry point that takes one:
the forward, the backward, the cache forward (split decode path) and the NVFP4-style forward,
each against the oracle called with the same scale.  Bar as for the default scale."""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, to_dev

pytestmark = pytest.mark.gpu


def bf16(a):
    return W.round_to_bf16(np.asarray(a, dtype=np.float64))


def quantize(q, k, v):
    import torch
    from bit_attention_amd import ops
    return (*ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0), *ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0),
            *ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1))


@pytest.mark.parametrize("scale,causal", [(0.3, True), (0.02, False)])
def test_forward_and_backward_custom_scale(scale, causal):
    import torch
    from bit_attention_amd import ops
    rng = np.random.default_rng(int(scale * 1000) + causal)
    B, Hq, Hkv, N, d = 1, 4, 2, 256, 128
    q = bf16(rng.standard_normal((B, Hq, N, d)))
    k = bf16(rng.standard_normal((B, Hkv, N, d)))
    v = bf16(rng.standard_normal((B, Hkv, N, d)))
    do = bf16(rng.standard_normal((B, Hq, N, d)) * 0.1)
    args = quantize(q, k, v)
    o, m, l = ops.attn_fp4_fwd(*args, causal=causal, softmax_scale=scale)
    dq, dk, dv = ops.attn_fp4_bwd_recompute(*args, o, to_dev(do, torch.bfloat16), m, l, causal=causal,
                                            softmax_scale=scale)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    o, m, l, dq, dk, dv = map(f, (o, m, l, dq, dk, dv))
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal, scale=scale)
    compare(o, ro, "O scale %g" % scale)
    assert np.max(np.abs(m - rm)) <= 1e-5 * max(1.0, np.abs(rm).max())
    compare_l(l, rl, "l scale %g" % scale)
    m_ref = oracle.attn_row_max(q, k, causal=causal, scale=scale)
    rq, rk, rv = oracle.attn_bwd(q, k, v, o, do, m_ref, l, causal=causal, scale=scale)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(g, r, "%s scale %g" % (name, scale))


def test_split_decode_custom_scale():
    import torch
    from bit_attention_amd import ops
    rng = np.random.default_rng(77)
    B, Hq, Hkv, Nk, d, scale = 2, 8, 2, 2048, 128, 0.25
    q = bf16(rng.standard_normal((B, Hq, 1, d)))
    kc = bf16(rng.standard_normal((B, Hkv, Nk, d)))
    vc = bf16(rng.standard_normal((B, Hkv, Nk, d)))
    lens = np.array([Nk, 1234], dtype=np.int32)
    assert ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, 1, Nk, d) > 0
    o, m, l = ops.attn_fp4_fwd_kvcache(*quantize(q, kc, vc), seqlens_k=to_dev(lens), causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attn_fwd_kvcache(q, kc, vc, lens, causal=True, scale=scale)
    compare(o.float().cpu().numpy(), ro, "decode O scale %g" % scale)
    assert np.max(np.abs(m.cpu().numpy() - rm)) <= 1e-5 * max(1.0, np.abs(rm).max())


def test_nvfp4_forward_custom_scale():
    import torch
    from bit_attention_amd import ops
    rng = np.random.default_rng(78)
    B, Hq, Hkv, N, d, scale = 1, 2, 1, 192, 64, 0.4
    q = bf16(rng.standard_normal((B, Hq, N, d)))
    k = bf16(rng.standard_normal((B, Hkv, N, d)))
    v = bf16(rng.standard_normal((B, Hkv, N, d)))
    nq = [ops.attn_fp4_nv_quantize(to_dev(x, torch.bfloat16), ax) for x, ax in ((q, 0), (k, 0), (v, 1))]
    o, m, l = ops.attn_fp4_nv_fwd(*nq[0], *nq[1], *nq[2], causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=True, scale=scale, fmt="nv")
    compare(o.float().cpu().numpy(), ro, "NVFP4 O scale %g" % scale)
    assert np.max(np.abs(m.cpu().numpy() - rm)) <= 1e-5 * max(1.0, np.abs(rm).max())
    compare_l(l.cpu().numpy(), rl, "NVFP4 l scale %g" % scale)
