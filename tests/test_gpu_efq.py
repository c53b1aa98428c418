"""GPU parity of the exp-free (EFQ) forward mode against the oracle's EFQ reading.

The oracle implements the stated reading of the EFQ-Softmax rule (oracle/efq.py); the pages give
no formula, so this checks the kernel against that reading.  Same bar as the exp-then-quantize
forward: rel-L2 <= 5e-3 and max-abs <= 3e-2 (plus the bf16 half-ulp) on O, m to fp32 precision,
l to the rel-L2 bar.  The distance to the exp-then-quantize oracle and the cosine against exact
attention are printed as context.
"""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, cosine, to_dev

pytestmark = pytest.mark.gpu


def gpu_fwd_efq(q, k, v, causal):
    import torch
    from bit_attention_amd import ops
    qc, qs = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    kc, ks = ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0)
    vc, vs = ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1)
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    m = torch.full((B, Hq, N), float("nan"), device="cuda")
    l = torch.full((B, Hq, N), float("nan"), device="cuda")
    o, m, l = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=causal, o=o, m=m, l=l, p_rule=ops.P_EFQ)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()


def check(o, m, l, ro, rm, rl, label):
    info = compare(o, ro, label + " O")
    assert np.max(np.abs(m - rm)) <= 1e-5 * max(1.0, np.abs(rm).max()), label
    compare_l(l, rl, label + " l")
    return info


def test_tiny_full():
    w = W.WORKLOADS["tiny_b1h2n256d64"]
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    o, m, l = gpu_fwd_efq(q, k, v, w.causal)
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=w.causal, p_rule="efq")
    info = check(o, m, l, ro, rm, rl, w.name)
    re, _, _ = oracle.attn_fwd(q, k, v, causal=w.causal, p_rule="exp")
    ex = oracle.softmax_attention(q, k, v)
    print("%s EFQ: rel-L2 %.3e; rel distance to exp-then-quantize %.3e; cosine(GPU, exact) %.5f" % (
        w.name, info["rel_l2"], np.linalg.norm(ro - re) / np.linalg.norm(re), cosine(o, ex)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,Hq,Hkv", [(64, 128, 1, 1), (192, 128, 4, 2), (128, 64, 3, 1)])
def test_small_shapes(N, d, Hq, Hkv, causal):
    rng = np.random.default_rng(300 + N + d + Hq + int(causal))
    q = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 1.3)
    k = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    o, m, l = gpu_fwd_efq(q, k, v, causal)
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal, p_rule="efq")
    check(o, m, l, ro, rm, rl, "N%d d%d Hq%d Hkv%d causal%d" % (N, d, Hq, Hkv, causal))


@pytest.mark.parametrize("name", ["llm_causal_b2h16n4096d128", "dit_b1h24n32768d128"])
def test_full_size_sampled_rows(name):
    w = W.WORKLOADS[name]
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    o, m, l = gpu_fwd_efq(q, k, v, w.causal)
    assert np.all(np.isfinite(o)) and np.all(l >= 1.0)
    rows = W.sample_rows(w.N, 96)
    for b, h in sorted({(0, 0), (w.B - 1, w.Hq - 1)}):
        g = h // (w.Hq // w.Hkv)
        args = (q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1])
        ro, rm, rl = oracle.attn_fwd(*args, causal=w.causal, rows=rows, p_rule="efq")
        info = check(o[b, h, rows], m[b, h, rows], l[b, h, rows], ro[0, 0], rm[0, 0], rl[0, 0],
                     "%s head (%d,%d)" % (name, b, h))
        re = oracle.attn_fwd(*args, causal=w.causal, rows=rows[:32], p_rule="exp")[0][0, 0]
        print("%s head (%d,%d) EFQ rel-L2 %.3e; rel distance to exp-then-quantize on 32 rows %.3e" % (
            name, b, h, info["rel_l2"], np.linalg.norm(o[b, h, rows[:32]] - re) / np.linalg.norm(re)))
