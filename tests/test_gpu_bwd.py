"""GPU parity of attn_fp4_bwd_recompute against the float64 oracle backward.

The oracle backward is fed the GPU forward's O (the D term is defined on the forward output that
is passed in) and l, and the exact row max of the quantized scores for m (the forward's final
running max, which the GPU saves rounded to fp32).  Bar: rel-L2 <= 5e-3 and max-abs <= 3e-2
(plus the half-ulp of the bf16 store) on dQ, dK and dV.  The full-size QAT workload runs in the
bench's launch configuration and is compared on sampled query rows (dQ) and sampled 32-key
blocks (dK, dV) of sampled heads.
"""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, cosine, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(q, k, v, do, causal):
    import torch
    from bit_attention_amd import ops
    qc, qs = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    kc, ks = ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0)
    vc, vs = ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1)
    o, m, l = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=causal)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nan = float("nan")
    dq = torch.full((B, Hq, N, d), nan, dtype=torch.bfloat16, device="cuda")
    dk = torch.full((B, Hkv, N, d), nan, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((B, Hkv, N, d), nan, dtype=torch.bfloat16, device="cuda")
    ws = torch.full((ops.attn_fp4_bwd_workspace_bytes(B, Hq, Hkv, N, d),), 0xFF, dtype=torch.uint8, device="cuda")
    ops.attn_fp4_bwd_recompute(qc, qs, kc, ks, vc, vs, o, to_dev(do, torch.bfloat16), m, l, causal=causal,
                               dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    return f(o), f(m), f(l), f(dq), f(dk), f(dv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,Hq,Hkv", [(64, 128, 1, 1), (192, 128, 4, 2), (256, 64, 2, 2), (128, 128, 2, 1),
                                        (256, 128, 4, 2), (384, 128, 2, 2), (256, 128, 8, 1), (192, 64, 2, 1)])
def test_small_shapes_full(N, d, Hq, Hkv, causal):
    rng = np.random.default_rng(100 + N + d + Hq + int(causal))
    q = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 1.5)
    k = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    do = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 0.1)
    o, m, l, dq, dk, dv = run_gpu(q, k, v, do, causal)
    m_ref = oracle.attn_row_max(q, k, causal=causal)
    assert np.max(np.abs(m - m_ref)) <= 1e-5 * max(1.0, np.abs(m_ref).max())
    rq, rk, rv = oracle.attn_bwd(q, k, v, o, do, m_ref, l, causal=causal)
    tag = "N%d d%d Hq%d Hkv%d causal%d" % (N, d, Hq, Hkv, causal)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        info = compare(g, r, tag + " " + name)
        print("%s %s rel-L2 %.3e" % (tag, name, info["rel_l2"]))


def test_zero_q_closed_form():
    """Q = 0: every P~ = 1 so A = 1/N, dV_j = mean_i dO_i; dK = 0 exactly."""
    rng = np.random.default_rng(5)
    N, d = 256, 128
    q = np.zeros((1, 2, N, d), dtype=np.float32)
    k = W.round_to_bf16(rng.standard_normal((1, 2, N, d)) * 3)
    v = W.round_to_bf16(rng.standard_normal((1, 2, N, d)))
    do = W.round_to_bf16(rng.standard_normal((1, 2, N, d)))
    o, m, l, dq, dk, dv = run_gpu(q, k, v, do, False)
    assert np.all(dk == 0)
    want = np.broadcast_to(do.astype(np.float64).mean(axis=2, keepdims=True), dv.shape)
    compare(dv, want, "Q=0 dV")
    rq, _, _ = oracle.attn_bwd(q, k, v, o, do, np.zeros((1, 2, N)), l)
    compare(dq, rq, "Q=0 dQ")


def test_qat_workload_full_size_sampled():
    w = W.WORKLOADS["qat_bwd_b1h16n8192d128"]
    q, k, v, do = (W.gen_tensor(w, t) for t in ("q", "k", "v", "do"))
    o, m, l, dq, dk, dv = run_gpu(q, k, v, do, w.causal)
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    rows = W.sample_rows(w.N, 96)
    blocks = np.array([0, 1, 77, 128, 200, w.N // 32 - 1])
    keys = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    for h in (0, w.Hq - 1):
        sl = slice(h, h + 1)
        m_ref = oracle.attn_row_max(q[:, sl], k[:, sl])
        rq, rk, rv = oracle.attn_bwd(q[:, sl], k[:, sl], v[:, sl], o[:, sl], do[:, sl], m_ref, l[:, sl],
                                     rows=rows, key_blocks=blocks)
        for name, g, r in (("dQ", dq[0, h, rows], rq[0, 0]), ("dK", dk[0, h, keys], rk[0, 0]),
                           ("dV", dv[0, h, keys], rv[0, 0])):
            info = compare(g, r, "qat head %d %s" % (h, name))
            print("qat head %d %s rel-L2 %.3e max-abs %.3e" % (h, name, info["rel_l2"], info["max_abs"]))
    # accuracy context: gradients of exact attention on the unquantized inputs (head 0, sampled rows)
    ex_o, ex_m, ex_l = oracle.attn_fwd(q[:, :1], k[:, :1], v[:, :1], quant=False)
    ex = oracle.attn_bwd(q[:, :1], k[:, :1], v[:, :1], ex_o, do[:, :1], ex_m, ex_l, quant=False, rows=rows,
                         key_blocks=blocks)
    print("qat cosine vs exact-attention gradients: dQ %.4f dK %.4f dV %.4f" % (
        cosine(dq[0, 0, rows], ex[0][0, 0]), cosine(dk[0, 0, keys], ex[1][0, 0]), cosine(dv[0, 0, keys], ex[2][0, 0])))


def test_causal_gqa_mid_size_sampled():
    """Causal GQA backward at a size with many query tiles per key block and key blocks past the
    first (the causal start tile, the walk over both query heads of a KV head): sampled query rows
    (dQ) and sampled 32-key blocks (dK, dV, summed over the group) against the oracle."""
    rng = np.random.default_rng(2048)
    B, Hq, Hkv, N, d = 1, 4, 2, 2048, 128
    q = W.round_to_bf16(rng.standard_normal((B, Hq, N, d)) * 1.2)
    k = W.round_to_bf16(rng.standard_normal((B, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_normal((B, Hkv, N, d)))
    do = W.round_to_bf16(rng.standard_normal((B, Hq, N, d)) * 0.1)
    o, m, l, dq, dk, dv = run_gpu(q, k, v, do, True)
    rows = W.sample_rows(N, 160)
    blocks = np.array([0, 3, 4, 5, 31, 32, 33, 47, 60, N // 32 - 1])
    keys = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    m_ref = oracle.attn_row_max(q, k, causal=True)
    rq, rk, rv = oracle.attn_bwd(q, k, v, o, do, m_ref, l, causal=True, rows=rows, key_blocks=blocks)
    for name, g, r in (("dQ", dq[:, :, rows], rq), ("dK", dk[:, :, keys], rk), ("dV", dv[:, :, keys], rv)):
        info = compare(g, r, "causal gqa N2048 " + name)
        print("causal gqa N2048 %s rel-L2 %.3e max-abs %.3e" % (name, info["rel_l2"], info["max_abs"]))


@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_deterministic(causal):
    """No atomics and fixed summation orders: two backward calls give identical bits."""
    rng = np.random.default_rng(41 + int(causal))
    N, d, Hq, Hkv = 256, 128, 4, 2
    q = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 1.5)
    k = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_normal((1, Hkv, N, d)))
    do = W.round_to_bf16(rng.standard_normal((1, Hq, N, d)) * 0.1)
    first = run_gpu(q, k, v, do, causal)
    second = run_gpu(q, k, v, do, causal)
    for name, a, b in zip(("o", "m", "l", "dq", "dk", "dv"), first, second):
        assert np.array_equal(a, b, equal_nan=True), name
