"""GPU parity of the NVFP4-style path (attn_fp4_nv_quantize, attn_fp4_nv_fwd) against the oracle.

Quantize: codes, E4M3 scales, the tensor scale G and the tensor amax are bit-exact (every rounding
step is fp32 round-to-nearest-even on both sides).  Forward: the bar of the MXFP4 forward (rel-L2
<= 5e-3, max-abs <= 3e-2 plus the bf16 store's half-ulp) on O, m to 1e-5 relative, l to the output
bar; full outputs at small sizes (several tiles, ragged 128-row tails, causal, GQA, d = 64 and 128,
all three workgroup shapes), sampled rows at the video and causal LLM sizes in the launch
configuration the bench times.
"""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def bf16(a):
    return W.round_to_bf16(np.asarray(a, dtype=np.float64))


def ref_quant(x, axis):
    """Oracle codes/scales/G in the library's layouts (axis 1: [.., d, n/2] codes, [.., d, n/16] scales)."""
    x = np.asarray(x, dtype=np.float64)
    g, amax = oracle.nv_tensor_scale(x)
    src = x if axis == 0 else np.swapaxes(x, -1, -2)
    c, s, _ = oracle.quantize_nv(src, axis=-1, g=g)
    return oracle.pack_nibbles(c, -1), s, g, amax


def gpu_quant(x, axis):
    import torch
    from bit_attention_amd import ops
    c, s, ts = ops.attn_fp4_nv_quantize(to_dev(x, torch.bfloat16), axis)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), ts.cpu().numpy()


def check_quant(x, axis, label):
    print(label, x.shape, "axis", axis, flush=True)
    gc, gs, gts = gpu_quant(x, axis)
    rc, rs, g, amax = ref_quant(x, axis)
    assert gts[0] == g, "%s: G %r != %r" % (label, gts[0], g)
    assert gts[1] == amax, "%s: amax %r != %r" % (label, gts[1], amax)
    assert np.array_equal(gs, rs), "%s: scales differ at %d places" % (label, int((gs != rs).sum()))
    assert np.array_equal(gc, rc), "%s: codes differ at %d bytes" % (label, int((gc != rc).sum()))


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("shape", [(2, 3, 256, 128), (1, 2, 144, 64), (1, 1, 16, 96), (3, 1, 400, 32)])
def test_quantize_bit_exact(shape, axis):
    if axis == 1 and shape[2] % 16:
        pytest.skip("axis 1 needs n % 16 == 0")
    rng = np.random.default_rng(hash((shape, axis)) % (1 << 32))
    # blocks spread over 2^-30 .. 1 of the tensor's largest: scales from 448 down to subnormal and 0
    x = rng.standard_normal(shape) * np.exp2(rng.uniform(-30, 0, shape[:-1] + (1,)))
    x.flat[rng.integers(x.size)] = 7.5
    check_quant(bf16(x), axis, "spread")
    y = rng.standard_normal(shape) * 3
    y[..., :5, :] = 0.0
    y[..., 5, :] = -0.0
    y[..., 6, :] = rng.choice([1e-38, -1e-39, 5e-41], size=shape[-1])   # bf16 subnormals and tiny
    check_quant(bf16(y), axis, "zeros and subnormals")


def test_quantize_zero_and_constant_tensors():
    z = np.zeros((1, 2, 64, 64))
    check_quant(z, 0, "zeros")
    check_quant(z, 1, "zeros")
    c = np.full((1, 1, 64, 64), -2.5)
    check_quant(c, 0, "constant")
    check_quant(c, 1, "constant")


def test_quantize_every_bf16_magnitude():
    # every finite bf16 magnitude in [2^-20, 2^20), in blocks of 16 consecutive values; the tensor
    # scale is set by 2^20, so the block scales span the E4M3 range and beyond
    u = np.arange(1 << 15, dtype=np.uint32) << 16
    f = u.view(np.float32).astype(np.float64)
    f = f[(f >= 2.0 ** -20) & (f < 2.0 ** 20)]
    f = f[: f.size // 1024 * 1024]
    sign = np.where(np.arange(f.size) % 3 == 0, -1.0, 1.0)
    x = (f * sign).reshape(1, 1, -1, 64)
    check_quant(x, 0, "all magnitudes")
    check_quant(x, 1, "all magnitudes (axis 1)")


def nv_gpu_fwd(q, k, v, causal, repeat=1):
    import torch
    from bit_attention_amd import ops
    qc, qs, qt = ops.attn_fp4_nv_quantize(to_dev(q, torch.bfloat16), 0)
    kc, ks, kt = ops.attn_fp4_nv_quantize(to_dev(k, torch.bfloat16), 0)
    vc, vs, vt = ops.attn_fp4_nv_quantize(to_dev(v, torch.bfloat16), 1)
    B, Hq, N, d = q.shape
    outs = []
    for _ in range(repeat):
        o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        m = torch.full((B, Hq, N), float("nan"), device="cuda")
        l = torch.full((B, Hq, N), float("nan"), device="cuda")
        o, m, l = ops.attn_fp4_nv_fwd(qc, qs, qt, kc, ks, kt, vc, vs, vt, causal=causal, o=o, m=m, l=l)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()))
    return outs if repeat > 1 else outs[0]


def check_fwd(q, k, v, causal, o, m, l, heads, rows, label):
    scales = tuple(oracle.nv_tensor_scale(t)[0] for t in (q, k, v))
    Hq, Hkv = q.shape[1], k.shape[1]
    for b, h in heads:
        g = h // (Hq // Hkv)
        ro, rm, rl = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], causal=causal,
                                     rows=rows, fmt="nv", nv_tensor_scales=scales)
        info = compare(o[b, h, rows], ro[0, 0], "%s O head (%d,%d)" % (label, b, h))
        assert np.max(np.abs(m[b, h, rows] - rm[0, 0])) <= 1e-5 * max(1.0, np.abs(rm).max()), label
        compare_l(l[b, h, rows], rl[0, 0], label + " l")
        print("%s head (%d,%d): rel-L2 %.3e max-abs %.3e" % (label, b, h, info["rel_l2"], info["max_abs"]),
              flush=True)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [
    (1, 2, 2, 256, 64, False),     # eight waves per workgroup
    (1, 2, 2, 256, 128, True),
    (1, 4, 2, 192, 128, False),    # N % 128 = 64: two waves per workgroup
    (1, 4, 2, 192, 128, True),
    (2, 4, 1, 384, 128, True),     # N % 256 = 128: four waves per workgroup
    (1, 2, 1, 64, 64, True),       # a single tile
])
def test_forward_full_parity(B, Hq, Hkv, N, d, causal):
    rng = np.random.default_rng(B * 1000 + Hq * 100 + N + d + causal)
    q = bf16(rng.standard_normal((B, Hq, N, d)) * 1.5)
    k = bf16(rng.standard_normal((B, Hkv, N, d)) * 1.5)
    v = bf16(rng.standard_normal((B, Hkv, N, d)))
    print("nv fwd", (B, Hq, Hkv, N, d, causal), flush=True)
    o, m, l = nv_gpu_fwd(q, k, v, causal)
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    check_fwd(q, k, v, causal, o, m, l, heads, np.arange(N), "nv %s" % ((B, Hq, Hkv, N, d, causal),))


def test_forward_q_zero_is_mean_of_v_and_deterministic():
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 2, 256, 128
    q = np.zeros((B, H, N, d))
    k = bf16(rng.standard_normal((B, H, N, d)))
    v = bf16(rng.standard_normal((B, H, N, d)))
    (o1, m1, l1), (o2, m2, l2) = nv_gpu_fwd(q, k, v, True, repeat=2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(m1, m2)
    gv = oracle.nv_tensor_scale(v)[0]
    vh = np.stack([oracle.fake_quant_nv(v[0, h], 0, gv) for h in range(H)])
    pref = np.cumsum(vh, axis=1) / np.arange(1, N + 1)[None, :, None]
    compare(o1[0], pref, "Q = 0 causal prefix mean")
    np.testing.assert_array_equal(l1[0], np.broadcast_to(np.arange(1, N + 1), (H, N)))
    np.testing.assert_array_equal(m1, 0.0)


@pytest.mark.parametrize("name", ["dit_b1h24n32768d128", "llm_causal_b2h16n4096d128"])
def test_forward_full_size_sampled(name):
    w = W.WORKLOADS[name]
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    print("nv fwd", name, flush=True)
    o, m, l = nv_gpu_fwd(q, k, v, w.causal)
    rows = W.sample_rows(w.N, count=256)
    heads = [(0, 0), (w.B - 1, w.Hq - 1)]
    check_fwd(q, k, v, w.causal, o, m, l, heads, rows, name)


def test_forward_workspace_reuse_and_smaller_second_call():
    # one workspace serves a large call and then a smaller one; the second must not see the first
    import torch
    from bit_attention_amd import ops
    rng = np.random.default_rng(12)
    big = [bf16(rng.standard_normal((1, 4, 512, 128))) for _ in range(3)]
    small = [bf16(rng.standard_normal((1, 2, 128, 128)) * 2) for _ in range(3)]
    ws = torch.empty(ops.attn_fp4_nv_fwd_workspace_bytes(1, 4, 4, 512, 128), dtype=torch.uint8, device="cuda")
    outs = []
    for q, k, v in (big, small):
        qq = ops.attn_fp4_nv_quantize(to_dev(q, torch.bfloat16), 0)
        kq = ops.attn_fp4_nv_quantize(to_dev(k, torch.bfloat16), 0)
        vq = ops.attn_fp4_nv_quantize(to_dev(v, torch.bfloat16), 1)
        o, m, l = ops.attn_fp4_nv_fwd(*qq, *kq, *vq, causal=False, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()))
    q, k, v = small
    check_fwd(q, k, v, False, *outs[1], [(0, 0), (0, 1)], np.arange(128), "second call")
