"""Pins for the NVFP4-style reading of the oracle (CPU only).

Each pin comes from outside the oracle's own code: the E4M3 bit-field
definition and hand-computed values, an independent formulation of E4M3
rounding (quantum of the binade plus numpy's banker's rounding), brute
force over the 127 finite non-negative E4M3 values, blocks built to be
exactly representable, power-of-two equivariance, the element error bound
of block scaling, and closed forms of the forward (Q = 0 gives the mean of
V^; identical keys give the same).
"""

import numpy as np
import pytest

from oracle import (
    E2M1_GRID,
    E4M3_POS,
    attn_fwd,
    decode_e4m3,
    dequantize_nv,
    e4m3_round_codes,
    fake_quant_nv,
    nv_p_fake_quant,
    nv_tensor_scale,
    quantize_nv,
    softmax_attention,
)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def to_bf16(a):
    """Round float64 values to bfloat16 (round half to even) and return them as float64."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def e4m3_round_quantum(t):
    """E4M3 rounding written a second way: binade quantum, then banker's rounding."""
    t = np.asarray(t, dtype=np.float64)
    _, k = np.frexp(np.where(t > 0, t, 1.0))          # t = f 2^k, f in [0.5, 1)
    q_exp = np.maximum(k - 1, -6) - 3                 # 3 mantissa bits; subnormal quantum 2^-9
    r = np.round(t / np.ldexp(1.0, q_exp)) * np.ldexp(1.0, q_exp)
    return np.minimum(r, 448.0)


def test_e4m3_decode_table():
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
            0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x78: 256.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in hand.items():
        assert decode_e4m3(b) == v, hex(b)
    assert np.all(np.diff(E4M3_POS) > 0) and E4M3_POS.size == 127
    # every value is an integer of at most 4 bits times a power of two
    for v in E4M3_POS[1:]:
        m, e = np.frexp(v)
        assert (m * 16) == int(m * 16)


def test_e4m3_round_matches_quantum_form_and_brute_force():
    rng = np.random.default_rng(0)
    mids = (E4M3_POS[1:] + E4M3_POS[:-1]) / 2
    t = np.concatenate([
        E4M3_POS, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        rng.uniform(0, 500, 20000), np.exp(rng.uniform(np.log(1e-5), np.log(600), 20000)),
        [0.0, 448.0, 460.0, 464.0, 1e6, 2.0 ** -10, np.nextafter(2.0 ** -10, 1)],
    ])
    codes = e4m3_round_codes(t)
    np.testing.assert_array_equal(decode_e4m3(codes), e4m3_round_quantum(t))
    # brute force: nearest value, ties to the even code
    sub = t[::7]
    dist = np.abs(sub[:, None] - E4M3_POS[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    np.testing.assert_array_equal(codes[::7], pick)


def test_tensor_scale_and_largest_element():
    rng = np.random.default_rng(1)
    x = to_bf16(rng.standard_normal((4, 64)) * 3)
    g, amax = nv_tensor_scale(x)
    assert amax == np.abs(x).max()
    assert g == np.float32(np.float32(amax) / np.float32(2688))
    c, s, _ = quantize_nv(x, axis=-1)
    i, j = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert decode_e4m3(s[i, j // 16]) == 448.0
    assert (c[i, j] & 7) == 7                      # magnitude 6
    assert ((c[i, j] & 8) != 0) == (x[i, j] < 0)


def test_identity_on_representable_blocks():
    # G = 2^k exactly when amax = 2688 * 2^k; a block of E2M1 values times S * 2^k is exact
    rng = np.random.default_rng(2)
    k = -3
    G = 2.0 ** k
    blocks = []
    for S in [448.0, 1.0, 1.125, 2.0 ** -9, 3.5, 240.0]:
        vals = rng.choice(E2M1_GRID, 16) * rng.choice([-1, 1], 16)
        vals[rng.integers(16)] = 6.0                # the block max is 6 S G
        blocks.append(vals * S * G)
    x = np.concatenate(blocks)[None, :]
    assert np.abs(x).max() == 6 * 448 * G
    c, s, g = quantize_nv(x)
    assert g == G
    np.testing.assert_array_equal(dequantize_nv(c, s, g), x)
    np.testing.assert_array_equal(fake_quant_nv(x), x)


def test_power_of_two_equivariance_and_sign():
    rng = np.random.default_rng(3)
    x = to_bf16(rng.standard_normal((3, 128)))
    c0, s0, g0 = quantize_nv(x)
    for k in (-20, -1, 4, 30):
        c, s, g = quantize_nv(x * 2.0 ** k)
        np.testing.assert_array_equal(c, c0)
        np.testing.assert_array_equal(s, s0)
        assert g == g0 * np.float32(2.0 ** k)
    c, s, g = quantize_nv(-x)
    np.testing.assert_array_equal(c, c0 ^ 8)
    np.testing.assert_array_equal(s, s0)


def test_element_error_bound_and_axis():
    rng = np.random.default_rng(4)
    x = to_bf16(rng.standard_normal((2, 48, 32)) * np.exp(rng.uniform(-4, 4, (2, 48, 1))))
    for axis in (1, 2):
        c, s, g = quantize_nv(x, axis=axis)
        xh = dequantize_nv(c, s, g, axis=axis)
        S = np.repeat(decode_e4m3(s), 16, axis=axis) * np.float64(g)
        # within a binade of E2M1 the step is at most a third of the magnitude, below 1 it is 0.5;
        # saturation at 6 can only lose what the E4M3 rounding of the scale lost (< 1/16)
        mag = np.abs(x) / S
        step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
        assert np.all(np.abs(x - xh) <= (step / 2 + mag / 16 + 1e-6) * S)
    # quantizing along axis 1 is quantizing the transposed tensor along its last axis
    c1, s1, _ = quantize_nv(x, axis=1)
    cT, sT, _ = quantize_nv(np.swapaxes(x, 1, 2), axis=-1)
    np.testing.assert_array_equal(np.swapaxes(c1, 1, 2), cT)
    np.testing.assert_array_equal(np.swapaxes(s1, 1, 2), sT)


def test_zero_and_tiny_blocks():
    x = np.zeros((1, 32))
    x[0, 5] = -0.0
    c, s, g = quantize_nv(x)
    assert g == np.float32(2.0 ** -117)
    assert np.all(s == 0) and c[0, 5] == 8 and np.all(np.delete(c[0], 5) == 0)
    # a block far below the tensor's largest one gets S = 0 and only sign codes
    y = np.zeros((1, 32))
    y[0, 0] = 2688.0
    y[0, 16:] = -1e-5
    c, s, g = quantize_nv(y)
    assert s[0, 1] == 0 and np.all(c[0, 16:] == 8)


def test_p_rule():
    rng = np.random.default_rng(5)
    p = rng.uniform(0, 1, (8, 64))
    p[:, ::16] = 1.0                                  # one row max per block
    pt = nv_p_fake_quant(p)
    np.testing.assert_array_equal(pt[:, ::16], 1.0)  # the maximum is exact
    # with S = 448 the values are the E2M1 grid over 6: the widest gap, 4/6 .. 6/6, bounds the error
    assert np.all(np.abs(pt - p) <= 1 / 6 + 1e-12)
    # grid points over 6 in a block whose max is 1 are kept exactly
    q = np.zeros((1, 16))
    q[0, :4] = [1.0, 0.5, 1 / 3, 1 / 6]
    np.testing.assert_allclose(nv_p_fake_quant(q)[0, :4], q[0, :4], rtol=0, atol=1e-15)
    # small blocks keep relative precision through their own scale
    r = np.full((1, 16), 1e-3)
    assert abs(nv_p_fake_quant(r)[0, 0] - 1e-3) <= 1e-3 / 16
    assert np.all(nv_p_fake_quant(np.zeros((2, 32))) == 0)


def test_forward_nv_closed_forms():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, N, d = 1, 4, 2, 128, 64
    q = to_bf16(rng.standard_normal((B, Hq, N, d)))
    k = to_bf16(rng.standard_normal((B, Hkv, N, d)))
    v = to_bf16(rng.standard_normal((B, Hkv, N, d)))
    # quantizers off: the format does not matter and the tile loop is textbook attention
    for causal in (False, True):
        O, _, _ = attn_fwd(q, k, v, causal=causal, quant=False, fmt="nv")
        np.testing.assert_allclose(O, softmax_attention(q, k, v, causal=causal), atol=1e-12)
    gv = nv_tensor_scale(v)[0]
    vh = np.stack([np.stack([fake_quant_nv(v[b, g], 0, gv) for g in range(Hkv)]) for b in range(B)])
    # Q = 0: every p is 1, every block scale 448, every P~ exactly 1 -> mean of V^ (causal: prefix mean)
    z = np.zeros_like(q)
    O, m, l = attn_fwd(z, k, v, quant=True, fmt="nv")
    np.testing.assert_allclose(O, np.repeat(vh.mean(axis=2, keepdims=True), 2, axis=1).repeat(N, axis=2),
                               atol=1e-12)
    np.testing.assert_array_equal(l, N)
    O, _, l = attn_fwd(z, k, v, causal=True, quant=True, fmt="nv")
    pref = np.cumsum(vh, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(O, np.repeat(pref, 2, axis=1), atol=1e-12)
    np.testing.assert_array_equal(l[0, 0], np.arange(1, N + 1))
    # identical keys give uniform scores: the same mean, whatever Q is
    kk = np.repeat(k[:, :, :1], N, axis=2)
    O, _, _ = attn_fwd(q, kk, v, quant=True, fmt="nv")
    np.testing.assert_allclose(O, np.repeat(vh.mean(axis=2, keepdims=True), 2, axis=1).repeat(N, axis=2),
                               atol=1e-12)
    # V -> 2^k V scales O exactly; sampled rows match the full result
    O1, m1, l1 = attn_fwd(q, k, v, quant=True, fmt="nv")
    O2, m2, l2 = attn_fwd(q, k, v * 8.0, quant=True, fmt="nv")
    np.testing.assert_array_equal(O2, 8.0 * O1)
    rows = np.array([0, 5, 64, 127])
    Os, ms, ls = attn_fwd(q, k, v, quant=True, fmt="nv", rows=rows)
    np.testing.assert_allclose(Os, O1[:, :, rows], rtol=0, atol=1e-13)   # BLAS summation order only
    np.testing.assert_allclose(ls, l1[:, :, rows], rtol=1e-13)
    # the quantizers are on, and the finer blocks and scales of this format lose less than MXFP4
    # on Gaussian inputs (rel-L2 to the textbook result: 0.195 against 0.255 on this seed)
    T = softmax_attention(q, k, v)
    Om, _, _ = attn_fwd(q, k, v, quant=True)
    err_nv, err_mx = (np.linalg.norm(o - T) / np.linalg.norm(T) for o in (O1, Om))
    assert 0.05 < err_nv < err_mx
    with pytest.raises(ValueError):
        attn_fwd(q, k, v, fmt="nv", p_rule="efq")
