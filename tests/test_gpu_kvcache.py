"""GPU parity of attn_fp4_fwd_kvcache (chunked prefill and decode against a quantized cache).

The oracle is `oracle.attn_fwd_kvcache`.  Bar as for attn_fp4_fwd: rel-L2 <= 5e-3 and max-abs
<= 3e-2 (plus the bf16 store's half-ulp) on O, m to fp32 precision, l to the rel-L2 bar.  Rows
that see no key must give exactly O = 0, m = -inf, l = 0.  With Nq = Nk = L the cache forward
must equal the plain forward bit for bit (same tiles, same per-row arithmetic, only the packing
of rows into waves differs).  The full-size decode and chunked-prefill workloads run in the
launch configuration the bench times and are compared on sampled heads and rows.
"""

import numpy as np
import pytest

import oracle
from bit_attention_amd import workloads as W
from helpers import compare, compare_l, to_dev

pytestmark = pytest.mark.gpu


def quantize_cache(q, kc, vc):
    import torch
    from bit_attention_amd import ops
    qq = ops.attn_fp4_quantize(to_dev(q, torch.bfloat16), 0)
    kq = ops.attn_fp4_quantize(to_dev(kc, torch.bfloat16), 0)
    vq = ops.attn_fp4_quantize(to_dev(vc, torch.bfloat16), 1)
    return (*qq, *kq, *vq)


def gpu_kv(q, kc, vc, seqlens, causal, p_rule=0):
    import torch
    from bit_attention_amd import ops
    args = quantize_cache(q, kc, vc)
    B, Hq, Nq, d = q.shape
    o = torch.full((B, Hq, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    m = torch.full((B, Hq, Nq), float("nan"), device="cuda")
    l = torch.full((B, Hq, Nq), float("nan"), device="cuda")
    sl = None if seqlens is None else to_dev(np.asarray(seqlens, dtype=np.int32))
    o, m, l = ops.attn_fp4_fwd_kvcache(*args, seqlens_k=sl, causal=causal, o=o, m=m, l=l, p_rule=p_rule)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()


def check(o, m, l, ro, rm, rl, label):
    empty = rl == 0
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(m[empty])) and np.all(l[empty] == 0.0), label
    full = ~empty
    assert np.array_equal(np.isneginf(m), np.isneginf(rm)), label
    info = compare(o[full], ro[full], label + " O")
    assert np.max(np.abs(m[full] - rm[full]), initial=0.0) <= 1e-5 * max(1.0, np.abs(rm[full]).max(initial=0.0)), label
    if full.any():
        compare_l(l[full], rl[full], label + " l")
    return info


def rand_bf16(shape, seed, scale=1.0):
    return W.round_to_bf16(np.random.default_rng(seed).standard_normal(shape) * scale)


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, seqlens, causal
    (2, 4, 2, 1, 256, 128, [256, 77], True),        # decode, ragged length
    (2, 8, 2, 37, 320, 64, [320, 100], True),       # ragged chunk, group of 4 packed
    (1, 4, 4, 130, 192, 128, [150], False),         # non-causal, rows past one workgroup
    (3, 2, 1, 8, 128, 128, [5, 0, 128], True),      # rows with no key, an empty cache
    (1, 32, 8, 64, 256, 128, None, True),           # 256 packed rows: four-wave workgroups
    (2, 2, 2, 3, 64, 64, [64, 1], False),           # one tile; a single valid key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_Nq%d_Nk%d_d%d_c%d" % (c[:6] + (c[7],)))
def test_small_full(case):
    B, Hq, Hkv, Nq, Nk, d, seqlens, causal = case
    seed = 7000 + sum(case[:6])
    q = rand_bf16((B, Hq, Nq, d), seed, 1.3)
    kc = rand_bf16((B, Hkv, Nk, d), seed + 1)
    vc = rand_bf16((B, Hkv, Nk, d), seed + 2)
    o, m, l = gpu_kv(q, kc, vc, seqlens, causal)
    ro, rm, rl = oracle.attn_fwd_kvcache(q, kc, vc, seqlens, causal=causal)
    info = check(o, m, l, ro, rm, rl, str(case))
    print("%s: rel-L2 %.3e" % (case, info["rel_l2"]))


def test_small_efq():
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 21, 256, 128
    q = rand_bf16((B, Hq, Nq, d), 7101, 1.3)
    kc = rand_bf16((B, Hkv, Nk, d), 7102)
    vc = rand_bf16((B, Hkv, Nk, d), 7103)
    seqlens = [200, 256]
    o, m, l = gpu_kv(q, kc, vc, seqlens, True, p_rule=1)
    ro, rm, rl = oracle.attn_fwd_kvcache(q, kc, vc, seqlens, causal=True, p_rule="efq")
    check(o, m, l, ro, rm, rl, "efq")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 2)])
def test_equals_plain_forward_bitwise(causal, Hq, Hkv):
    import torch
    from bit_attention_amd import ops
    B, N, d = 1, 384, 128
    q = rand_bf16((B, Hq, N, d), 7200 + Hq, 1.5)
    k = rand_bf16((B, Hkv, N, d), 7201)
    v = rand_bf16((B, Hkv, N, d), 7202)
    args = quantize_cache(q, k, v)
    o1, m1, l1 = ops.attn_fp4_fwd(*args, causal=causal)
    o2, m2, l2 = ops.attn_fp4_fwd_kvcache(*args, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2) and torch.equal(l1, l2)


def test_decode_full_size_sampled_heads():
    w = W.CACHE_WORKLOADS["decode_b8hq32hkv8nk32768d128"]
    q = W.gen_cache_tensor(w, "q")
    kc, vc = W.gen_cache_tensor(w, "k"), W.gen_cache_tensor(w, "v")
    seqlens = W.cache_lengths(w)
    o, m, l = gpu_kv(q, kc, vc, seqlens, w.causal)
    assert np.all(np.isfinite(o)) and np.all(l >= 1.0)
    G = w.Hq // w.Hkv
    for b, g in [(0, 0), (3, 5), (w.B - 1, w.Hkv - 1)]:
        hs = slice(g * G, (g + 1) * G)
        ro, rm, rl = oracle.attn_fwd_kvcache(q[b:b + 1, hs], kc[b:b + 1, g:g + 1], vc[b:b + 1, g:g + 1],
                                             seqlens[b:b + 1], causal=w.causal)
        info = check(o[b:b + 1, hs], m[b:b + 1, hs], l[b:b + 1, hs], ro, rm, rl, "decode (%d, kv %d)" % (b, g))
        print("decode b%d kv%d L=%d: rel-L2 %.3e" % (b, g, seqlens[b], info["rel_l2"]))


def test_prefill_chunk_full_size_sampled_rows():
    w = W.CACHE_WORKLOADS["prefill_chunk_b1hq32hkv8nq2048nk32768d128"]
    q = W.gen_cache_tensor(w, "q")
    kc, vc = W.gen_cache_tensor(w, "k"), W.gen_cache_tensor(w, "v")
    seqlens = W.cache_lengths(w)
    o, m, l = gpu_kv(q, kc, vc, seqlens, w.causal)
    assert np.all(np.isfinite(o)) and np.all(l >= 1.0)
    rows = W.sample_rows(w.Nq, 48, edge=8)
    G = w.Hq // w.Hkv
    for h in (0, w.Hq - 1):
        g = h // G
        ro, rm, rl = oracle.attn_fwd_kvcache(q[:, h:h + 1], kc[:, g:g + 1], vc[:, g:g + 1], seqlens,
                                             causal=w.causal, rows=rows)
        info = check(o[:, h:h + 1, rows], m[:, h:h + 1, rows], l[:, h:h + 1, rows], ro, rm, rl,
                     "prefill chunk head %d" % h)
        print("prefill chunk head %d: rel-L2 %.3e" % (h, info["rel_l2"]))


SPLIT_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, seqlens, causal, p_rule
    (2, 8, 2, 1, 1024, 128, [1000, 333], True, 0),     # decode, ragged lengths
    (1, 4, 1, 37, 2048, 64, [1500], True, 0),          # short chunk, d = 64
    (2, 2, 2, 5, 512, 128, [512, 0], False, 0),        # an empty cache
    (3, 4, 4, 3, 1024, 128, [2, 700, 1024], True, 0),  # rows with no key next to full ones
    (2, 8, 2, 2, 1024, 128, [900, 1024], True, 1),     # EFQ
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_Nq%d_Nk%d_d%d_c%d_r%d" % (c[:6] + c[7:]))
def test_split_small_full(case):
    import torch
    from bit_attention_amd import ops
    B, Hq, Hkv, Nq, Nk, d, seqlens, causal, rule = case
    assert ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d) > 0, "the split path must run"
    seed = 7300 + sum(case[:6])
    q = rand_bf16((B, Hq, Nq, d), seed, 1.3)
    kc = rand_bf16((B, Hkv, Nk, d), seed + 1)
    vc = rand_bf16((B, Hkv, Nk, d), seed + 2)
    o, m, l = gpu_kv(q, kc, vc, seqlens, causal, p_rule=rule)
    ro, rm, rl = oracle.attn_fwd_kvcache(q, kc, vc, seqlens, causal=causal, p_rule="efq" if rule else "exp")
    info = check(o, m, l, ro, rm, rl, "split " + str(case))
    print("split %s: rel-L2 %.3e" % (case, info["rel_l2"]))
    # against the one-pass kernel: the same running maxima (so the same P~ codes), m bit for bit;
    # O and l differ only by the fp32 summation order
    args = quantize_cache(q, kc, vc)
    sl = to_dev(np.asarray(seqlens, dtype=np.int32))
    o1, m1, l1 = ops.attn_fp4_fwd_kvcache(*args, seqlens_k=sl, causal=causal, p_rule=rule, workspace=None)
    torch.cuda.synchronize()
    assert np.array_equal(m1.cpu().numpy(), m)
    np.testing.assert_allclose(l1.cpu().numpy(), l, rtol=1e-5, atol=0)
    np.testing.assert_allclose(o1.float().cpu().numpy(), o, rtol=1e-2, atol=1e-3)


def test_split_workspace_reuse_and_smaller_call():
    """The caller's workspace keeps the last call's contents: a second, smaller call must not
    read stale partial results."""
    import torch
    from bit_attention_amd import ops
    B, Hq, Hkv, Nk, d = 4, 8, 2, 2048, 128
    need = ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, 2, Nk, d)   # the larger call
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for Nq, seqlens, seed in ((2, [2048, 1900, 1000, 64], 7400), (1, [300, 2048, 7, 1024], 7401)):
        q = rand_bf16((B, Hq, Nq, d), seed, 1.3)
        kc = rand_bf16((B, Hkv, Nk, d), seed + 1)
        vc = rand_bf16((B, Hkv, Nk, d), seed + 2)
        args = quantize_cache(q, kc, vc)
        sl = to_dev(np.asarray(seqlens, dtype=np.int32))
        wsz = ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
        assert 0 < wsz <= need
        o, m, l = ops.attn_fp4_fwd_kvcache(*args, seqlens_k=sl, causal=True, workspace=ws[:wsz])
        torch.cuda.synchronize()
        ro, rm, rl = oracle.attn_fwd_kvcache(q, kc, vc, seqlens, causal=True)
        check(o.float().cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), ro, rm, rl, "reuse Nq=%d" % Nq)


def test_split_bitwise_deterministic():
    """The split path merges its ranges in a fixed order: two calls give identical bits."""
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 1, 4096, 128
    seqlens = [4096, 2500]
    q = rand_bf16((B, Hq, Nq, d), 7500, 1.3)
    kc = rand_bf16((B, Hkv, Nk, d), 7501)
    vc = rand_bf16((B, Hkv, Nk, d), 7502)
    from bit_attention_amd import ops
    assert ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, Nq, Nk, d) > 0, "the split path must run"
    first = gpu_kv(q, kc, vc, seqlens, True)
    second = gpu_kv(q, kc, vc, seqlens, True)
    for name, a, b in zip(("o", "m", "l"), first, second):
        assert np.array_equal(a, b), name
