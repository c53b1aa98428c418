"""Pins for the MXFP4 quantizer of the oracle (CPU only).

Each pin comes from somewhere other than the oracle's own code: the E2M1
grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} and its bit-field definition, brute force
over every finite bfloat16 value, a library rounding routine, closed forms
of the scale rule, and algebraic invariants of block scaling.
"""

import numpy as np
import pytest

from oracle import (
    E2M1_GRID,
    decode_e2m1,
    dequantize_mx,
    e2m1_round_codes,
    fake_quant_mx,
    pack_nibbles,
    quantize_mx,
    unpack_nibbles,
)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def all_finite_bf16():
    """Every finite bfloat16 value (both zeros included) as float64."""
    u = np.arange(1 << 16, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def brute_force_code(v):
    """Nearest grid magnitude by exhaustive distance; a tie goes to the even code index."""
    a = np.abs(v)[:, None]
    dist = np.abs(a - E2M1_GRID[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer an even index (mantissa bit 0)
    idx = np.arange(8)[None, :]
    score = np.where(cand, np.where(idx % 2 == 0, 0, 1) * 16 + idx, 999)
    mag = np.argmin(score, axis=1)
    return (mag | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def banker_round_value(v):
    """E2M1 rounding via numpy's round-half-to-even on the grid's step size."""
    a = np.abs(v)
    # grid step: 0.5 below 2, then 2**(k-1) in [2**k, 2**(k+1))
    k = np.floor(np.log2(np.maximum(a, 1.0)))
    step = np.where(a < 2.0, 0.5, 2.0 ** (k - 1))
    q = np.minimum(np.round(a / step) * step, 6.0)
    return np.copysign(q, v)


def test_decode_table_matches_grid_and_bitfields():
    literal = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = decode_e2m1(np.arange(16))
    assert got.tolist() == literal
    assert np.signbit(got[8]) and not np.signbit(got[0])
    # E2M1 bit fields: sign | exp(2) | mantissa(1), bias 1, exponent 0 is subnormal
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        val = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert got[c] == (-val if s else val)


def test_element_rule_exhaustive_bf16_against_brute_force():
    x = all_finite_bf16()
    # apply the element rule at several scale offsets so that every code region is hit
    for shift in range(-6, 3):
        v = x * 2.0 ** shift
        v = v[np.abs(v) < 16]
        ours = e2m1_round_codes(v)
        assert np.array_equal(ours, brute_force_code(v))
        assert np.array_equal(decode_e2m1(ours), banker_round_value(v))


def test_element_rule_ties_and_saturation_literals():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.0001, 6.0, 7.99, 100.0, -0.25, -0.1, -0.0, 0.0])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0, 6.0, -0.0, -0.0, -0.0, 0.0]
    got = decode_e2m1(e2m1_round_codes(v))
    assert got.tolist() == want
    assert np.array_equal(np.signbit(got), np.signbit(np.array(want)))


@pytest.mark.parametrize("anchor", [4.0, 6.0, 7.96875])
def test_quantize_exhaustive_bf16_with_anchored_blocks(anchor):
    """Every finite bf16 x placed in a block whose max is anchor*2**e fixes the scale at e."""
    x = all_finite_bf16()
    ok_total = 0
    for delta in range(0, 5):
        # choose e so that x / 2**e lies in [4, 8) / 2**delta, i.e. every magnitude band
        with np.errstate(divide="ignore"):
            ex = np.floor(np.log2(np.abs(x)))
        e = ex - 2 + delta
        keep = np.isfinite(e) & (e >= -127) & (e <= 125) & (np.abs(x) <= anchor * 2.0 ** e)
        xs, es = x[keep], e[keep]
        block = np.zeros((xs.shape[0], 32))
        block[:, 0] = anchor * 2.0 ** es
        block[:, 1] = xs
        block[:, 2] = -xs / 2
        codes, scales = quantize_mx(block, axis=-1)
        assert np.array_equal(scales[:, 0].astype(np.int64), (es + 127).astype(np.int64))
        v = xs / 2.0 ** es
        assert np.array_equal(codes[:, 1], brute_force_code(v))
        assert np.array_equal(codes[:, 2], brute_force_code(-v / 2))
        assert np.all(codes[:, 3:] == 0)
        ok_total += xs.shape[0]
    assert ok_total > 100000


def test_scale_rule_closed_form_from_float32_exponent_field():
    rng = np.random.default_rng(5)
    for dist in range(4):
        if dist == 0:
            x = rng.standard_normal((4096, 32))
        elif dist == 1:
            x = rng.standard_t(3, (4096, 32)) * 1e3
        elif dist == 2:
            x = rng.uniform(0, 1, (4096, 32)) * 2.0 ** rng.integers(-120, 120, (4096, 1))
        else:
            # block maxima exactly at, just below and just above powers of two
            p = 2.0 ** rng.integers(-100, 100, (4096, 1)).astype(np.float64)
            x = rng.uniform(-0.5, 0.5, (4096, 32)) * p
            x[:, 7] = p[:, 0] * np.array([1.0, 1 - 2.0 ** -8, 1 + 2.0 ** -7, 1.0])[np.arange(4096) % 4]
        x = x.astype(np.float32).astype(np.float64)
        _, s = quantize_mx(x, axis=-1)
        amax = np.abs(x).max(axis=1).astype(np.float32)
        field = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64)   # biased fp32 exponent
        want = np.clip(field - 127 - 2, -127, 127) + 127
        assert np.array_equal(s[:, 0].astype(np.int64), want)


def test_zero_and_tiny_blocks():
    z = np.zeros((2, 32))
    z[1, 5] = -0.0
    z[1, 6] = -0.0
    c, s = quantize_mx(z)
    assert np.all(s == 0)
    assert c[0].tolist() == [0] * 32
    assert c[1, 5] == 8 and c[1, 6] == 8
    # amax below the smallest normal: scale byte 0 (e = -127), values divided by 2**-127
    t = np.zeros((1, 32))
    t[0, 0] = 2.0 ** -130
    t[0, 1] = 3 * 2.0 ** -128
    c, s = quantize_mx(t)
    assert s[0, 0] == 0
    assert decode_e2m1(c[0, :2]).tolist() == [0.0, 1.5]


def test_identity_on_representable_blocks():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, (2000, 32))
    top = rng.choice([6, 7], size=2000)          # magnitude 4 or 6 present -> scale fixed at e
    codes[:, 0] = top
    e = rng.integers(-100, 100, 2000)
    x = decode_e2m1(codes) * 2.0 ** e[:, None]
    assert np.array_equal(fake_quant_mx(x), x)
    c2, s2 = quantize_mx(x)
    assert np.array_equal(s2[:, 0].astype(np.int64), e + 127)
    # codes equal up to the sign of zero (a -0 code may come back as -0: same bits)
    assert np.array_equal(c2, codes.astype(np.uint8))


def test_sign_power_of_two_equivariance_and_idempotence():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((3000, 64)) * 3).astype(np.float32).astype(np.float64)
    c, s = quantize_mx(x)
    for k in (-5, 1, 7):
        ck, sk = quantize_mx(x * 2.0 ** k)
        assert np.array_equal(ck, c)
        assert np.array_equal(sk.astype(np.int64), s.astype(np.int64) + k)
    cn, sn = quantize_mx(-x)
    assert np.array_equal(cn, c ^ 8)
    assert np.array_equal(sn, s)
    fq = fake_quant_mx(x)
    assert np.array_equal(fake_quant_mx(fq), fq)


def test_axis_argument_matches_transpose():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 96))
    c0, s0 = quantize_mx(x, axis=0)
    c1, s1 = quantize_mx(x.T, axis=-1)
    assert np.array_equal(c0, c1.T) and np.array_equal(s0, s1.T)
    assert np.array_equal(dequantize_mx(c0, s0, axis=0), dequantize_mx(c1, s1, axis=-1).T)


def test_worked_example_by_hand():
    # amax 0.9 -> floor(log2 0.9) = -1 -> e = -3 (byte 124); x / 2**-3 = 7.2, 0.8, -2.4, 4, 0.36
    # -> 6 (saturated), 1, -2, 4, 0.5
    x = np.zeros(32)
    x[:5] = [0.9, 0.1, -0.3, 0.5, 0.045]
    c, s = quantize_mx(x)
    assert s.tolist() == [124]
    assert c[:5].tolist() == [7, 2, 12, 6, 1]
    assert dequantize_mx(c, s)[:5].tolist() == [0.75, 0.125, -0.25, 0.5, 0.0625]


def test_pack_nibble_order():
    codes = np.array([[1, 2, 3, 4, 15, 8]], dtype=np.uint8)
    p = pack_nibbles(codes)
    assert p.tolist() == [[0x21, 0x43, 0x8F]]
    assert np.array_equal(unpack_nibbles(p), codes)
