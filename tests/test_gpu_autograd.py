"""The autograd wrapper: gradients land on Q, K, V and equal the direct backward entry point's.

The wrapper only marshals arguments, so its outputs must be bit-identical to calling
attn_fp4_quantize / attn_fp4_fwd / attn_fp4_bwd_recompute directly; one case is also compared with
the float64 oracle backward to the usual bar.
"""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,Hq,Hkv", [(128, 128, 2, 1), (192, 64, 2, 2)])
def test_autograd_matches_entry_points(N, d, Hq, Hkv, causal):
    import torch
    from bit_attention_amd import ops
    from bit_attention_amd.autograd import fp4_attention
    rng = np.random.default_rng(7 + N + d + int(causal))
    q = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)))
    k = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    do = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 0.1)
    tq, tk, tv = (to_dev(x, torch.bfloat16).requires_grad_(True) for x in (q, k, v))
    o = fp4_attention(tq, tk, tv, causal=causal)
    o.backward(to_dev(do, torch.bfloat16))
    # the same computation through the entry points
    qc, qs = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    kc, ks = ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0)
    vc, vs = ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1)
    o2, m2, l2 = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=causal)
    dq2, dk2, dv2 = ops.attn_fp4_bwd_recompute(qc, qs, kc, ks, vc, vs, o2, to_dev(do, torch.bfloat16), m2, l2,
                                               causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for name, a, b in (("dQ", tq.grad, dq2), ("dK", tk.grad, dk2), ("dV", tv.grad, dv2)):
        assert a is not None and a.shape == b.shape and a.dtype == torch.bfloat16, name
        assert torch.equal(a, b), name
    if not causal and d == 128:
        f = lambda t: t.float().cpu().numpy()
        m_ref = oracle.attn_row_max(q, k, causal=causal)
        rq, rk, rv = oracle.attn_bwd(q, k, v, f(o2), do, m_ref, f(l2), causal=causal)
        for name, g, r in (("dQ", tq.grad, rq), ("dK", tk.grad, rk), ("dV", tv.grad, rv)):
            compare(f(g), r, "autograd " + name)
