"""Pins for the oracle's cache forward `attn_fwd_kvcache` (CPU only).

The new rows are the last Nq positions of each sequence; the cache holds L_b valid keys and
values of a larger capacity.  Pins: with the quantizers off, textbook softmax attention over the
visible keys with bottom-right causal alignment (the library formula on the sliced sequence);
with them on and L_b a multiple of the 32-token V block, the rows of the full forward at those
positions; Q = 0 gives the mean of V^ over the visible keys with V^ quantized over the capacity
(ragged L_b); rows that see no key give O = 0, m = -inf, l = 0; cache contents past L_b (whole
V blocks) do not matter.
"""

import numpy as np
import pytest

from oracle import attn_fwd, attn_fwd_kvcache, fake_quant_mx, softmax_attention


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def caches(B, Hkv, Nk, d, seed):
    return rand((B, Hkv, Nk, d), seed, 1.3), rand((B, Hkv, Nk, d), seed + 1)


@pytest.mark.parametrize("causal", [False, True])
def test_unquantized_equals_textbook(causal):
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 5, 192, 32
    q = rand((B, Hq, Nq, d), 11, 1.5)
    k, v = caches(B, Hkv, Nk, d, 12)
    seqlens = np.array([192, 70, 5])
    o, m, l = attn_fwd_kvcache(q, k, v, seqlens, causal=causal, quant=False)
    for b, L in enumerate(seqlens):
        # the sequence of length L whose last Nq rows are the new queries
        q_full = np.zeros((1, Hq, L, d))
        q_full[0, :, L - Nq:] = q[b]
        ref = softmax_attention(q_full, k[b:b + 1, :, :L], v[b:b + 1, :, :L], causal=causal)[0, :, L - Nq:]
        assert np.max(np.abs(o[b] - ref)) < 1e-12
        s = np.einsum("hnd,hmd->hnm", q[b], np.repeat(k[b, :, :L], 2, axis=0)) / np.sqrt(d)
        if causal:
            s = np.where(np.arange(L)[None, :] <= (L - Nq + np.arange(Nq))[:, None], s, -np.inf)
        assert np.allclose(m[b], s.max(-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq", [1, 7, 64])
def test_rows_of_the_full_forward(causal, Nq):
    B, Hq, Hkv, Nk, d = 2, 2, 1, 256, 64
    k, v = caches(B, Hkv, Nk, d, 21)
    seqlens = np.array([256, 160])                   # multiples of 32
    q = rand((B, Hq, Nq, d), 22, 2.0)
    o, m, l = attn_fwd_kvcache(q, k, v, seqlens, causal=causal)
    for b, L in enumerate(seqlens):
        Lt = -(-L // 64) * 64                        # the full forward needs whole tiles
        q_full = np.zeros((1, Hq, Lt, d))
        q_full[0, :, L - Nq:L] = q[b]
        kk, vv = k[b:b + 1, :, :Lt].copy(), v[b:b + 1, :, :Lt].copy()
        rows = np.arange(L - Nq, L)
        if Lt > L:
            if not causal:
                continue                             # non-causal would see keys past L
            vv[:, :, L:] = 0.0                       # whole blocks past L: no effect on V^
        ro, rm, rl = attn_fwd(q_full, kk, vv, causal=causal, rows=rows)
        assert np.array_equal(o[b], ro[0]) and np.array_equal(m[b], rm[0]) and np.array_equal(l[b], rl[0])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_v_hat_over_the_capacity(causal):
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 2, 6, 128, 32
    k, v = caches(B, Hkv, Nk, d, 31)
    seqlens = np.array([77, 10])                     # ragged: V^ blocks straddle the length
    q = np.zeros((B, Hq, Nq, d))
    o, m, l = attn_fwd_kvcache(q, k, v, seqlens, causal=causal)
    for b, L in enumerate(seqlens):
        for h in range(Hq):
            v_hat = fake_quant_mx(v[b, h], axis=0)   # over the capacity, blocks from position 0
            for i in range(Nq):
                n = (L - Nq + i + 1) if causal else L
                assert l[b, h, i] == n and m[b, h, i] == 0.0
                assert np.allclose(o[b, h, i], v_hat[:n].mean(axis=0), rtol=0, atol=1e-12)


def test_rows_that_see_no_key():
    B, Hq, Hkv, Nq, Nk, d = 2, 1, 1, 8, 64, 32
    k, v = caches(B, Hkv, Nk, d, 41)
    q = rand((B, Hq, Nq, d), 42)
    o, m, l = attn_fwd_kvcache(q, k, v, np.array([3, 0]), causal=True)
    # L = 3 < Nq: rows 0..4 sit at negative positions; L = 0: every row is empty
    empty = np.zeros((B, Nq), bool)
    empty[0, :5] = True
    empty[1, :] = True
    assert np.all(o[:, 0][empty] == 0.0) and np.all(np.isneginf(m[:, 0][empty])) and np.all(l[:, 0][empty] == 0.0)
    assert np.all(l[:, 0][~empty] >= 1.0) and np.all(np.isfinite(o[:, 0][~empty]))
    o2, m2, l2 = attn_fwd_kvcache(q, k, v, np.array([0, 0]), causal=False)
    assert np.all(o2 == 0.0) and np.all(np.isneginf(m2)) and np.all(l2 == 0.0)


def test_cache_past_the_length_does_not_matter():
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 4, 256, 64
    k, v = caches(B, Hkv, Nk, d, 51)
    q = rand((B, Hq, Nq, d), 52, 1.5)
    L = 100
    ref = attn_fwd_kvcache(q, k, v, np.array([L]), causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = rand(k2[:, :, L:].shape, 53, 50.0)        # any keys past L
    v2[:, :, 128:] = rand(v2[:, :, 128:].shape, 54, 50.0)    # whole V blocks past L
    got = attn_fwd_kvcache(q, k2, v2, np.array([L]), causal=True)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


def test_rejects_bad_arguments():
    k, v = caches(1, 1, 64, 32, 61)
    q = rand((1, 1, 2, 32), 62)
    with pytest.raises(ValueError):
        attn_fwd_kvcache(q, k, v, np.array([65]))
    with pytest.raises(ValueError):
        attn_fwd_kvcache(q, k[:, :, :48], v[:, :, :48])
