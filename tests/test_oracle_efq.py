"""Pins of the EFQ-Softmax code rule (oracle/efq.py), a reading of the EFQ-Softmax abstract.

The pages give no formula, so these pin the oracle to the stated reading and to its relation
with exp-then-quantize, not to numbers printed on the pages.
"""

import numpy as np

import oracle


def block(values):
    x = np.full(32, -np.inf)
    x[: len(values)] = values
    return x


def test_fitted_line_closed_form():
    # least squares of k against u = log2 v_k: slope = cov(u, k) / var(u), intercept = mean(k) - slope mean(u)
    u = np.log2(np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]))
    k = np.arange(1.0, 8.0)
    slope = ((u - u.mean()) * (k - k.mean())).sum() / ((u - u.mean()) ** 2).sum()
    assert abs(oracle.EFQ_A - slope) < 1e-12
    assert abs(oracle.EFQ_B - (k.mean() - slope * u.mean())) < 1e-12
    assert abs(oracle.EFQ_A - 1.747056609226127) < 1e-12 and abs(oracle.EFQ_B - 2.314118449252336) < 1e-12


def test_integer_points_map_to_that_code():
    # block max x = 0 (p = 1) -> e = -2 and y = x + 2; A y + B = k exactly -> code k
    for k in range(0, 8):
        y = (k - oracle.EFQ_B) / oracle.EFQ_A
        if y > 2.0:                # not below the block max (y = 2 there)
            continue
        for dy in (0.0, 0.2 / oracle.EFQ_A, -0.2 / oracle.EFQ_A):
            codes, e = oracle.efq_codes(block([0.0, y + dy - 2.0]))
            assert e[0] == -2.0
            assert codes[1] == k, (k, dy, codes[1])


def test_half_way_points_round_half_even():
    tested = 0
    for k in range(0, 5):
        x = (k + 0.5 - oracle.EFQ_B) / oracle.EFQ_A - 2.0     # block max 0 -> y = x + 2
        if oracle.EFQ_A * (x + 2.0) + oracle.EFQ_B != k + 0.5:  # use only exact half-way points
            continue
        codes, _ = oracle.efq_codes(block([0.0, x]))
        want = k if k % 2 == 0 else k + 1
        assert codes[1] == want, (k, codes[1])
        tested += 1
    assert tested >= 2


def test_block_max_power_of_two_is_exact():
    # the block maximum p = 2^j: e = j - 2, y = 2, A 2 + B = 5.81 -> code 6 (4.0): P~ = 4 * 2^(j - 2) = p
    for j in (0, -1, -7, -30):
        vals = oracle.efq_fake_quant(block([float(j), float(j) - 0.3]))
        assert vals[0] == 2.0 ** j

def test_monotone_and_within_one_step_of_exp_then_quantize():
    x = np.linspace(-9.0, 0.0, 32 * 4001)
    x = np.sort(x)[::-1].reshape(-1, 32)
    x[:, 0] = 0.0                                     # every block has p_max = 1
    codes, e = oracle.efq_codes(x)
    exact, _ = oracle.quantize_mx(np.exp2(x), axis=-1)
    flat = codes.reshape(-1)
    xs = x.reshape(-1)
    order = np.argsort(xs)
    assert np.all(np.diff(flat[order]) >= 0)           # monotone in x
    assert np.max(np.abs(codes - exact)) <= 1
    assert np.mean(codes == exact) > 0.5


def test_masked_block_is_zero():
    codes, e = oracle.efq_codes(np.full(32, -np.inf))
    assert np.all(codes == 0) and e[0] == -127.0


def test_zero_q_gives_mean_of_v_hat():
    rng = np.random.default_rng(3)
    q = np.zeros((1, 2, 128, 64))
    k = rng.standard_normal((1, 2, 128, 64))
    v = rng.standard_normal((1, 2, 128, 64))
    o, m, l = oracle.attn_fwd(q, k, v, p_rule="efq")
    vh = oracle.fake_quant_mx(v, axis=-2)
    assert np.allclose(o, np.broadcast_to(vh.mean(axis=2, keepdims=True), o.shape), rtol=1e-13, atol=1e-13)
    assert np.allclose(l, 128.0)
    oc, _, _ = oracle.attn_fwd(q, k, v, causal=True, p_rule="efq")
    want = np.cumsum(vh, axis=2) / np.arange(1, 129)[None, None, :, None]
    assert np.allclose(oc, want, rtol=1e-12, atol=1e-12)


def test_efq_close_to_exp_then_quantize_attention():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 1, 256, 64)) for _ in range(3))
    oe, _, _ = oracle.attn_fwd(q, k, v, p_rule="exp")
    of, _, _ = oracle.attn_fwd(q, k, v, p_rule="efq")
    ref = oracle.softmax_attention(q, k, v)
    cos = lambda a, b: float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum()))
    # both are 4-bit approximations of softmax attention; the exp-free codes stay close
    assert cos(oe, ref) > 0.96 and cos(of, ref) > 0.95
    assert np.linalg.norm(of - oe) / np.linalg.norm(oe) < 0.3
