"""GPU parity of attn_fp4_fwd against the float64 oracle.

Bar: rel-L2 <= 5e-3 and max-abs <= 3e-2 (plus the half-ulp of the final bf16 store) on O; the
saved m and l against the oracle's.  Full-size workloads run in the same launch configuration the
bench times and are compared on sampled rows of sampled heads (rows are independent, so each
sampled row is exact parity).  Cosine similarity against exact float64 softmax attention on the
unquantized inputs is printed as accuracy context (not a gate).
"""

import dataclasses

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, cosine, to_dev

pytestmark = pytest.mark.gpu


def quantize_all(q, k, v):
    import torch
    from bit_attention_amd import ops
    qc, qs = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    kc, ks = ops.attn_fp4_quantize(to_dev(k, torch.bfloat16), 0)
    vc, vs = ops.attn_fp4_quantize(to_dev(v, torch.bfloat16), 1)
    return qc, qs, kc, ks, vc, vs


def gpu_fwd(q, k, v, causal, poison=True):
    import torch
    from bit_attention_amd import ops
    ops_in = quantize_all(q, k, v)
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.bfloat16, device="cuda") if poison else None
    m = torch.full((B, Hq, N), float("nan"), device="cuda") if poison else None
    l = torch.full((B, Hq, N), float("nan"), device="cuda") if poison else None
    o, m, l = ops.attn_fp4_fwd(*ops_in, causal=causal, o=o, m=m, l=l)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()


def check_rows(w, q, k, v, o, m, l, heads, rows, label):
    for b, h in heads:
        g = h // (w.Hq // w.Hkv)
        ro, rm, rl = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                     causal=w.causal, rows=rows)
        info = compare(o[b, h, rows], ro[0, 0], "%s O head (%d,%d)" % (label, b, h))
        assert np.max(np.abs(m[b, h, rows] - rm[0, 0])) <= 1e-5 * max(1.0, np.abs(rm).max()), label
        # l = the sum of the same P~ codes, accumulated in fp32 with the history rescales; held
        # element-wise to 1e-4 relative (fp32 accumulation over 512 tiles stays near 2e-5)
        compare_l(l[b, h, rows], rl[0, 0], label + " l")
        print("%s head (%d,%d): rel-L2 %.3e max-abs %.3e" % (label, b, h, info["rel_l2"], info["max_abs"]))


def test_tiny_full_parity_and_cosine():
    w = W.WORKLOADS["tiny_b1h2n256d64"]
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    o, m, l = gpu_fwd(q, k, v, w.causal)
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=w.causal)
    info = compare(o, ro, w.name)
    assert np.max(np.abs(m - rm)) < 1e-5
    compare_l(l, rl, w.name + " l")
    ex = oracle.softmax_attention(q, k, v)
    print("%s: rel-L2 %.3e max-abs %.3e cosine(GPU, exact attention) %.5f cosine(oracle, exact) %.5f" % (
        w.name, info["rel_l2"], info["max_abs"], cosine(o, ex), cosine(ro, ex)))


@pytest.mark.parametrize("name", ["llm_causal_b2h16n4096d128", "dit_b1h24n32768d128",
                                  "gqa_causal_b1hq32hkv8n16384d128", "qat_bwd_b1h16n8192d128"])
def test_full_size_workloads_sampled_rows(name):
    w = W.WORKLOADS[name]
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    o, m, l = gpu_fwd(q, k, v, w.causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(m)) and np.all(l >= 1.0)
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (0, w.Hq // 2 + 1)})
    rows = W.sample_rows(w.N, 96 if w.N > 8192 else 160)
    check_rows(w, q, k, v, o, m, l, heads, rows, name)
    # accuracy context on a few rows: cosine against exact attention (unquantized inputs)
    b, h = heads[0]
    g = h // (w.Hq // w.Hkv)
    rr = rows[:32]
    ex = oracle.attn_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], causal=w.causal,
                         rows=rr, quant=False)[0][0, 0]
    print("%s: cosine(GPU, exact attention) on %d rows = %.5f" % (name, rr.size, cosine(o[b, h, rr], ex)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,Hq,Hkv", [(64, 128, 1, 1), (192, 128, 4, 2), (128, 64, 3, 1), (320, 64, 2, 2),
                                        (256, 128, 8, 1), (192, 64, 8, 2)])
def test_small_shapes_full(N, d, Hq, Hkv, causal):
    rng = np.random.default_rng(N + d + Hq + int(causal))
    q = W.round_to_bf16(rng.standard_normal((2, Hq, N, d)) * 1.5)
    k = W.round_to_bf16(rng.standard_normal((2, Hkv, N, d)))
    v = W.round_to_bf16(rng.standard_t(4, (2, Hkv, N, d)))
    o, m, l = gpu_fwd(q, k, v, causal)
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal)
    compare(o, ro, "N%d d%d Hq%d Hkv%d causal%d" % (N, d, Hq, Hkv, causal))


def _tile_max_rises(q, k, causal, bc=64):
    """Fraction of (row, visible key tile after the first) at which the running max of the
    quantized scores rises (CPU, from the oracle's quantizer)."""
    qh = oracle.fake_quant_mx(q.astype(np.float64), axis=-1)[0, 0]
    kh = oracle.fake_quant_mx(k.astype(np.float64), axis=-1)[0, 0]
    s = qh @ kh.T
    N = s.shape[0]
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    tmax = s.reshape(N, N // bc, bc).max(axis=2)
    run = np.maximum.accumulate(tmax, axis=1)
    rises = run[:, 1:] > run[:, :-1]
    visible = np.arange(1, N // bc)[None, :] * bc <= np.arange(N)[:, None] if causal else np.ones_like(rises)
    return float(rises[visible].mean())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["rising", "falling"])
def test_history_rescale_on_every_tile_or_none(order, causal):
    """Scores that rise along the keys make nearly every key tile raise every row's running max, so
    the history rescale runs on each tile with alpha < 1; scores that fall leave the max where the
    first tile put it, so the rescale never runs after it.  Both against the oracle; the per-tile
    maxima are checked on the CPU first, so that the inputs do what they are meant to."""
    rng = np.random.default_rng(23 + int(causal) + 2 * (order == "rising"))
    N, d, H = 2048, 128, 2
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    t = np.linspace(0.5, 12.0, N) if order == "rising" else np.linspace(12.0, 0.5, N)
    k = W.round_to_bf16(t[None, None, :, None] * u * np.sqrt(d) + 0.05 * rng.standard_normal((1, H, N, d)))
    q = W.round_to_bf16((1.0 + 0.2 * rng.random((1, H, N, 1))) * u + 0.05 * rng.standard_normal((1, H, N, d)))
    v = W.round_to_bf16(rng.standard_normal((1, H, N, d)))
    frac = _tile_max_rises(q[:, :1], k[:, :1], causal)
    print("%s causal=%d: running max rises at %.3f of the visible tiles" % (order, causal, frac))
    assert (frac > 0.95) if order == "rising" else (frac < 0.02)
    o, m, l = gpu_fwd(q, k, v, causal)
    ro, rm, rl = oracle.attn_fwd(q, k, v, causal=causal)
    info = compare(o, ro, "%s causal=%d" % (order, causal))
    assert np.max(np.abs(m - rm)) <= 1e-5 * max(1.0, np.abs(rm).max())
    compare_l(l, rl, "%s causal=%d l" % (order, causal))
    print("%s causal=%d: rel-L2 %.3e max-abs %.3e" % (order, causal, info["rel_l2"], info["max_abs"]))


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_quantized_v(causal):
    """Closed form: Q = 0 -> every P~ = 1, O_i = mean of V^ rows (causal: prefix mean), l_i = count."""
    rng = np.random.default_rng(7)
    N, d = 256, 128
    q = np.zeros((1, 2, N, d), dtype=np.float32)
    k = W.round_to_bf16(rng.standard_normal((1, 2, N, d)) * 4)
    v = W.round_to_bf16(rng.standard_normal((1, 2, N, d)))
    o, m, l = gpu_fwd(q, k, v, causal)
    vh = oracle.fake_quant_mx(v.astype(np.float64), axis=-2)
    if causal:
        want = np.cumsum(vh, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        assert np.array_equal(l, np.broadcast_to(np.arange(1, N + 1, dtype=np.float32), l.shape))
    else:
        want = np.broadcast_to(vh.mean(axis=2, keepdims=True), vh.shape)
        assert np.all(l == N)
    assert np.all(m == 0)
    compare(o, want, "Q=0 causal=%d" % causal)


@pytest.mark.parametrize("H,N", [(8, 14336), (8, 12288), (3, 1024)])
def test_causal_work_orders_cover_every_row(H, N):
    """The causal launch orders its row blocks per XCD: mixed first rounds when an XCD holds three
    to four row blocks per CU (N = 14336 and 12288 with 8 heads), longest first otherwise (3 heads
    do not spread evenly over the 8 XCDs).  Every row must be written (outputs start as NaN) and
    sampled rows of the first and last head must match the oracle."""
    rng = np.random.default_rng(N + H)
    q = W.round_to_bf16(rng.standard_normal((1, H, N, 128)) * 1.5)
    k = W.round_to_bf16(rng.standard_normal((1, H, N, 128)))
    v = W.round_to_bf16(rng.standard_normal((1, H, N, 128)))
    o, m, l = gpu_fwd(q, k, v, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(m)) and np.all(l >= 1.0)
    rows = W.sample_rows(N, 48, edge=8)
    for h in (0, H - 1):
        ro, rm, rl = oracle.attn_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], causal=True, rows=rows)
        compare(o[0, h, rows], ro[0, 0], "causal H%d N%d head %d" % (H, N, h))
        compare_l(l[0, h, rows], rl[0, 0], "causal H%d N%d head %d l" % (H, N, h))


def test_bitwise_deterministic():
    import torch
    from bit_attention_amd import ops
    w = dataclasses.replace(W.WORKLOADS["gqa_causal_b1hq32hkv8n16384d128"], Hq=8, Hkv=2, N=2048)
    q, k, v = (W.gen_tensor(w, t) for t in "qkv")
    args = quantize_all(q, k, v)
    a = ops.attn_fp4_fwd(*args, causal=True)
    b = ops.attn_fp4_fwd(*args, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_invalid_arguments_raise():
    import torch
    from bit_attention_amd import ops
    rng = np.random.default_rng(1)
    x = W.round_to_bf16(rng.standard_normal((1, 2, 96, 128)))
    args = quantize_all(x, x, x)
    with pytest.raises(ops.AttnFp4Error) as e:
        ops.attn_fp4_fwd(*args)                      # N = 96 is not a multiple of 64
    assert e.value.status == 1
    torch.cuda.synchronize()
