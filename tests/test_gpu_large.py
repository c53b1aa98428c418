"""Parity at the largest sizes this suite runs: a 131072-token head through the forward (MXFP4 and
NVFP4-style), a 32768-token GQA group through the backward, a 131072-key decode through the split
cache forward, and a 2^27-element quantization (both formats), each launched whole and compared
with the oracle on sampled rows, heads or blocks (rows, heads and blocks are independent, so each
sample is exact parity)."""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, to_dev

pytestmark = pytest.mark.gpu


def rand_bf16(shape, seed, scale=1.0):
    return W.round_to_bf16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * scale)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_131072_tokens_sampled_rows(causal):
    import torch
    from bit_attention_amd import ops
    N, d = 131072, 128
    q = rand_bf16((1, 1, N, d), 8100 + causal, 1.2)
    k = rand_bf16((1, 1, N, d), 8102)
    v = rand_bf16((1, 1, N, d), 8103)
    args = (*ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0), *ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0),
            *ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1))
    o, m, l = ops.attn_fp4_fwd(*args, causal=causal)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 4095, 65536, 99999, N - 65, N - 2, N - 1])
    o = o[0, 0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    m = m[0, 0].cpu().numpy()[rows]
    l = l[0, 0].cpu().numpy()[rows]
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal, rows=rows)
    compare(o, ro[0, 0], "N=131072 O")
    assert np.max(np.abs(m - rm[0, 0])) <= 1e-5 * max(1.0, np.abs(rm).max())
    compare_l(l, rl[0, 0], "N=131072 l")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_32768_tokens_gqa_sampled(causal):
    """The backward over two query heads sharing one KV head at N = 32768 (512 key tiles per query
    row, 256 key blocks per head): dQ on sampled query rows, dK and dV (summed over the two query
    heads) on sampled 32-key blocks, against the oracle fed the GPU forward's O and l."""
    from test_gpu_bwd import run_gpu
    N, d = 32768, 128
    q = rand_bf16((1, 2, N, d), 8300 + causal, 1.2)
    k = rand_bf16((1, 1, N, d), 8302)
    v = rand_bf16((1, 1, N, d), 8303)
    do = rand_bf16((1, 2, N, d), 8304, 0.1)
    o, m, l, dq, dk, dv = run_gpu(q, k, v, do, causal)
    rows = np.array([0, 1, 63, 64, 4095, 16384, 29999, N - 65, N - 2, N - 1])
    blocks = np.array([0, 1, 255, 256, 511, 700, N // 32 - 2, N // 32 - 1])
    keys = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    m_ref = oracle.attn_row_max(q, k, causal=causal)
    rq, rk, rv = oracle.attn_bwd(q, k, v, o, do, m_ref, l, causal=causal, rows=rows, key_blocks=blocks)
    for name, g, r in (("dQ", dq[:, :, rows], rq), ("dK", dk[:, :, keys], rk), ("dV", dv[:, :, keys], rv)):
        info = compare(g, r, "N=32768 backward causal=%d %s" % (causal, name))
        print("N=32768 backward causal=%d %s rel-L2 %.3e max-abs %.3e" % (causal, name, info["rel_l2"],
                                                                          info["max_abs"]))


def test_decode_131072_keys_split():
    import torch
    from bit_attention_amd import ops
    B, Hq, Hkv, Nk, d = 2, 8, 2, 131072, 128
    assert ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, 1, Nk, d) > 0
    q = rand_bf16((B, Hq, 1, d), 8110, 1.3)
    kc = rand_bf16((B, Hkv, Nk, d), 8111)
    vc = rand_bf16((B, Hkv, Nk, d), 8112)
    seqlens = np.array([Nk, 77777], dtype=np.int32)
    args = (*ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0), *ops.attn_fp4_quantize(to_dev(kc, torch.bfloat16), 0),
            *ops.attn_fp4_quantize(to_dev(vc, torch.bfloat16), 1))
    o, m, l = ops.attn_fp4_fwd_kvcache(*args, seqlens_k=to_dev(seqlens), causal=True)
    torch.cuda.synchronize()
    o, m, l = o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    for b, g in [(0, 1), (1, 0)]:
        hs = slice(4 * g, 4 * g + 4)
        ro, rm, rl = oracle.attn_fwd_kvcache(q[b:b + 1, hs], kc[b:b + 1, g:g + 1], vc[b:b + 1, g:g + 1],
                                             seqlens[b:b + 1], causal=True)
        compare(o[b:b + 1, hs], ro, "decode Nk=131072 O (%d,%d)" % (b, g))
        assert np.max(np.abs(m[b:b + 1, hs] - rm)) <= 1e-5 * max(1.0, np.abs(rm).max())
        compare_l(l[b:b + 1, hs], rl, "decode l")


@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_2_27_elements_sampled(axis):
    import torch
    from bit_attention_amd import ops
    bh, n, d = 8, 131072, 128                         # 2^27 elements
    x = torch.randn(bh, n, d, device="cuda", dtype=torch.float32).mul_(3.0).to(torch.bfloat16)
    c, s = ops.attn_fp4_quantize(x, axis)
    torch.cuda.synchronize()
    r = np.random.default_rng(8120 + axis)
    for h in r.choice(bh, 2, replace=False):
        blk = int(r.integers(0, n // 32 - 64))
        rows = slice(32 * blk, 32 * blk + 2048)       # 64 whole blocks of 32 tokens
        xs = x[h, rows].float().cpu().numpy()
        if axis == 0:
            rc, rs = oracle.quantize_mx(xs, axis=-1)
            assert np.array_equal(s[h, rows].cpu().numpy(), rs)
            assert np.array_equal(c[h, rows].cpu().numpy(), oracle.pack_nibbles(rc, -1))
        else:
            rc, rs = oracle.quantize_mx(xs.T, axis=-1)                      # [d, 2048]
            packed = oracle.pack_nibbles(rc, -1).reshape(d, 64, 16).swapaxes(0, 1)   # [64 blocks, d, 16]
            assert np.array_equal(s[h, blk:blk + 64].cpu().numpy(), rs.T)
            assert np.array_equal(c[h, blk:blk + 64].cpu().numpy(), packed)


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_nvfp4_forward_131072_tokens_sampled_rows(d, causal):
    # the NVFP4-style path at the same length: tensor scales over the whole tensors, sampled rows
    import torch
    from bit_attention_amd import ops
    N = 131072
    q = rand_bf16((1, 1, N, d), 8200 + d + causal, 1.2)
    k = rand_bf16((1, 1, N, d), 8202)
    v = rand_bf16((1, 1, N, d), 8203)
    qq, kq, vq = (ops.attn_fp4_nv_quantize(to_dev(x, torch.bfloat16), ax) for x, ax in ((q, 0), (k, 0), (v, 1)))
    o, m, l = ops.attn_fp4_nv_fwd(*qq, *kq, *vq, causal=causal)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 4095, 65536, 99999, N - 65, N - 2, N - 1])
    o = o[0, 0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    m = m[0, 0].cpu().numpy()[rows]
    l = l[0, 0].cpu().numpy()[rows]
    scales = tuple(oracle.nv_tensor_scale(t)[0] for t in (q, k, v))
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal, rows=rows, fmt="nv", nv_tensor_scales=scales)
    compare(o, ro[0, 0], "NVFP4 N=131072 O")
    assert np.max(np.abs(m - rm[0, 0])) <= 1e-5 * max(1.0, np.abs(rm).max())
    compare_l(l, rl[0, 0], "NVFP4 N=131072 l")


@pytest.mark.parametrize("axis", [0, 1])
def test_nvfp4_quantize_2_27_elements_sampled(axis):
    # the tensor scale comes from the whole 2^27-element tensor (amax on the device, checked here
    # against the host's); codes and scales of sampled 2048-token slices are bit-exact
    import torch
    from bit_attention_amd import ops
    bh, n, d = 8, 131072, 128
    x = torch.randn(bh, n, d, device="cuda", dtype=torch.float32).mul_(3.0).to(torch.bfloat16)
    c, s, ts = ops.attn_fp4_nv_quantize(x, axis)
    torch.cuda.synchronize()
    amax = float(x.abs().max().float().cpu())
    g, _ = oracle.nv_tensor_scale(np.array([amax]))
    tsh = ts.cpu().numpy()
    assert tsh[1] == np.float32(amax) and tsh[0] == g
    r = np.random.default_rng(8130 + axis)
    for h in r.choice(bh, 2, replace=False):
        blk = int(r.integers(0, n // 16 - 128))
        rows = slice(16 * blk, 16 * blk + 2048)       # 128 whole blocks of 16 tokens
        xs = x[h, rows].float().cpu().numpy()
        if axis == 0:
            rc, rs, _ = oracle.quantize_nv(xs, axis=-1, g=g)
            assert np.array_equal(s[h, rows].cpu().numpy(), rs)
            assert np.array_equal(c[h, rows].cpu().numpy(), oracle.pack_nibbles(rc, -1))
        else:
            rc, rs, _ = oracle.quantize_nv(xs.T, axis=-1, g=g)              # [d, 2048]
            assert np.array_equal(s[h, :, blk:blk + 128].cpu().numpy(), rs)
            assert np.array_equal(c[h, :, 8 * blk:8 * blk + 1024].cpu().numpy(), oracle.pack_nibbles(rc, -1))
