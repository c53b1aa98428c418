"""Pins for the oracle's fake-quantized attention forward and backward (CPU only).

Pins: textbook softmax attention (quantizers off) for any tile width, causal
and GQA; a single-tile direct formula and a two-tile unrolled formula with
the quantizers on; closed forms (Q = 0 gives the mean of V^, identical V^
rows give that row); exact power-of-two scaling in V; float64 autograd of
textbook attention and central finite differences for the backward.
"""

import numpy as np
import pytest
import torch

from oracle import attn_bwd, attn_fwd, attn_row_max, fake_quant_mx, softmax_attention


def rand(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    # bf16-like values are not required by the oracle; plain float64 normals
    return r.standard_normal(shape) * scale


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bc", [16, 64, 256])
def test_unquantized_equals_textbook(causal, bc):
    q, k, v = rand((1, 4, 256, 32), 1, 1.5), rand((1, 2, 256, 32), 2, 1.5), rand((1, 2, 256, 32), 3)
    o, m, l = attn_fwd(q, k, v, causal=causal, bc=bc, quant=False)
    ref = softmax_attention(q, k, v, causal=causal)
    assert np.max(np.abs(o - ref)) < 1e-12
    # m is the row max of the scaled scores, l the row sum of exp(s - m)
    s = np.einsum("bhnd,bhmd->bhnm", q, np.repeat(k, 2, axis=1)) / np.sqrt(32)
    if causal:
        s = np.where(np.tril(np.ones((256, 256), bool)), s, -np.inf)
    assert np.allclose(m, s.max(-1), rtol=0, atol=1e-12)
    assert np.allclose(l, np.exp(s - s.max(-1, keepdims=True)).sum(-1), rtol=1e-12)


def test_single_tile_direct_formula():
    q, k, v = rand((1, 1, 64, 64), 4, 2.0), rand((1, 1, 64, 64), 5), rand((1, 1, 64, 64), 6)
    o, m, l = attn_fwd(q, k, v)
    qh, kh = fake_quant_mx(q[0, 0], -1), fake_quant_mx(k[0, 0], -1)
    vh = fake_quant_mx(v[0, 0], 0)
    s = qh @ kh.T / 8.0
    pt = fake_quant_mx(np.exp(s - s.max(1, keepdims=True)), -1)
    want = (pt @ vh) / pt.sum(1, keepdims=True)
    assert np.max(np.abs(o[0, 0] - want)) < 1e-13
    assert np.allclose(l[0, 0], pt.sum(1), rtol=1e-14)


def test_two_tile_unrolled_history():
    """Tile 0 is quantized against its own max; tile 1 raises the max; the history is rescaled."""
    q = rand((1, 1, 128, 32), 7)
    k = rand((1, 1, 128, 32), 8)
    k[0, 0, 64:] *= 3.0        # second tile tends to hold the larger scores
    v = rand((1, 1, 128, 32), 9)
    o, m, l = attn_fwd(q, k, v, bc=64)
    qh, kh, vh = fake_quant_mx(q[0, 0]), fake_quant_mx(k[0, 0]), fake_quant_mx(v[0, 0], 0)
    s = qh @ kh.T / np.sqrt(32)
    s0, s1 = s[:, :64], s[:, 64:]
    m0 = s0.max(1)
    m1 = np.maximum(m0, s1.max(1))
    p0 = fake_quant_mx(np.exp(s0 - m0[:, None]))
    p1 = fake_quant_mx(np.exp(s1 - m1[:, None]))
    a = np.exp(m0 - m1)
    num = a[:, None] * (p0 @ vh[:64]) + p1 @ vh[64:]
    den = a * p0.sum(1) + p1.sum(1)
    assert np.max(np.abs(o[0, 0] - num / den[:, None])) < 1e-13
    assert np.allclose(m[0, 0], m1, rtol=1e-14, atol=0)
    # the history matters: quantizing tile 0 against the final max gives a different result
    p0_late = fake_quant_mx(np.exp(s0 - m1[:, None]))
    alt = (p0_late @ vh[:64] + p1 @ vh[64:]) / (p0_late.sum(1) + p1.sum(1))[:, None]
    assert np.max(np.abs(alt - num / den[:, None])) > 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_quantized_v(causal):
    N = 256
    q = np.zeros((1, 2, N, 64))
    k = rand((1, 2, N, 64), 10, 3.0)
    v = rand((1, 2, N, 64), 11, 2.0)
    o, m, l = attn_fwd(q, k, v, causal=causal)
    for h in range(2):
        vh = fake_quant_mx(v[0, h], 0)
        if causal:
            want = np.cumsum(vh, axis=0) / np.arange(1, N + 1)[:, None]
            assert np.array_equal(l[0, h], np.arange(1, N + 1, dtype=np.float64))
        else:
            want = np.broadcast_to(vh.mean(0), (N, 64))
            assert np.all(l[0, h] == N)
        assert np.max(np.abs(o[0, h] - want) / (np.abs(want) + 1e-300)) < 1e-13
        assert np.all(m[0, h] == 0)


def test_identical_v_rows_give_that_row():
    N = 192
    c = np.array([0.5, -1.5, 3.0, 0.0] * 8)          # representable in every channel's block
    v = np.broadcast_to(c, (1, 1, N, 32)).copy()
    o, _, _ = attn_fwd(rand((1, 1, N, 32), 12, 2.0), rand((1, 1, N, 32), 13, 2.0), v, causal=True)
    assert np.allclose(o[0, 0], np.broadcast_to(c, (N, 32)), rtol=1e-14, atol=0)


def test_power_of_two_scaling_of_v_is_exact():
    q, k, v = rand((1, 2, 128, 64), 14), rand((1, 2, 128, 64), 15), rand((1, 2, 128, 64), 16)
    o, _, _ = attn_fwd(q, k, v)
    for s in (-3, 4):
        o2, _, _ = attn_fwd(q, k, v * 2.0 ** s)
        assert np.array_equal(o2, o * 2.0 ** s)


def test_row_sampling_matches_full():
    q, k, v = rand((1, 4, 256, 32), 17), rand((1, 2, 256, 32), 18), rand((1, 2, 256, 32), 19)
    rows = np.array([0, 5, 63, 64, 130, 255])
    for causal in (False, True):
        full = attn_fwd(q, k, v, causal=causal)
        part = attn_fwd(q, k, v, causal=causal, rows=rows)
        for a, b in zip(full, part):
            assert np.array_equal(a[:, :, rows], b)


def torch_attention_grads(q, k, v, do, causal, scale=None):
    tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    B, Hq, N, d = q.shape
    group = Hq // k.shape[1]
    kk = tk.repeat_interleave(group, dim=1)
    vv = tv.repeat_interleave(group, dim=1)
    s = torch.matmul(tq, kk.transpose(-1, -2).contiguous()) * (scale or 1.0 / np.sqrt(d))
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_unquantized_equals_autograd(causal):
    q, k, v = rand((1, 4, 128, 32), 20), rand((1, 2, 128, 32), 21), rand((1, 2, 128, 32), 22)
    do = rand((1, 4, 128, 32), 23)
    o, m, l = attn_fwd(q, k, v, causal=causal, quant=False)
    dq, dk, dv = attn_bwd(q, k, v, o, do, m, l, causal=causal, quant=False, chunk=48)
    _, gq, gk, gv = torch_attention_grads(q, k, v, do, causal)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert np.max(np.abs(a - b)) < 1e-10


def test_backward_unquantized_finite_differences():
    q, k, v = rand((1, 1, 64, 16), 24), rand((1, 1, 64, 16), 25), rand((1, 1, 64, 16), 26)
    do = rand((1, 1, 64, 16), 27)
    o, m, l = attn_fwd(q, k, v, quant=False)
    dq, dk, dv = attn_bwd(q, k, v, o, do, m, l, quant=False)

    def loss(q_, k_, v_):
        return float(np.sum(softmax_attention(q_, k_, v_) * do))

    h = 1e-6
    rng = np.random.default_rng(28)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in (1, 1, 64, 16))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-6


def test_backward_zero_q_equals_autograd_at_quantized_point():
    """Q = 0 makes every score equal, so P~ = p exactly and the STE gradient is exact."""
    N = 128
    q = np.zeros((1, 2, N, 64))
    k, v = rand((1, 2, N, 64), 29, 2.0), rand((1, 2, N, 64), 30)
    do = rand((1, 2, N, 64), 31)
    o, m, l = attn_fwd(q, k, v)
    dq, dk, dv = attn_bwd(q, k, v, o, do, m, l)
    kh = fake_quant_mx(k, -1)
    vh = np.swapaxes(fake_quant_mx(np.swapaxes(v, -1, -2), -1), -1, -2)
    ro, gq, gk, gv = torch_attention_grads(q, kh, vh, do, False)
    assert np.max(np.abs(o - ro)) < 1e-13
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert np.max(np.abs(a - b)) < 1e-12


def test_backward_dk_sums_to_zero_unquantized():
    """Shift invariance of softmax over keys: the dK rows of one head sum to zero."""
    q, k, v = rand((1, 1, 128, 32), 32), rand((1, 1, 128, 32), 33), rand((1, 1, 128, 32), 34)
    do = rand((1, 1, 128, 32), 35)
    o, m, l = attn_fwd(q, k, v, quant=False)
    _, dk, _ = attn_bwd(q, k, v, o, do, m, l, quant=False)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-11


def test_backward_sampling_matches_full():
    q, k, v = rand((1, 2, 128, 32), 36), rand((1, 1, 128, 32), 37), rand((1, 1, 128, 32), 38)
    do = rand((1, 2, 128, 32), 39)
    o, m, l = attn_fwd(q, k, v)
    full = attn_bwd(q, k, v, o, do, m, l, chunk=40)
    rows = np.array([1, 64, 127])
    kb = np.array([3, 0])
    part = attn_bwd(q, k, v, o, do, m, l, rows=rows, key_blocks=kb)
    keys = np.concatenate([np.arange(0, 32), np.arange(96, 128)])
    assert np.allclose(part[0], full[0][:, :, rows], rtol=0, atol=1e-14)
    assert np.allclose(part[1], full[1][:, :, keys], rtol=0, atol=1e-14)
    assert np.allclose(part[2], full[2][:, :, keys], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_row_max_equals_forward_final_max(causal):
    q, k, v = rand((1, 4, 192, 32), 40, 2.0), rand((1, 2, 192, 32), 41), rand((1, 2, 192, 32), 42)
    _, m, _ = attn_fwd(q, k, v, causal=causal)
    assert np.array_equal(attn_row_max(q, k, causal=causal, chunk=50), m)


def _fq_torch(x, axis):
    """MXFP4 fake quantization of a float64 tensor's values (the oracle's quantizer, pinned in
    tests/test_oracle_mx.py), as a constant: gradients are attached by the caller."""
    return torch.from_numpy(fake_quant_mx(x.detach().numpy(), axis))


def _ste(x, axis):
    # straight-through estimator: forward value Q(x), gradient of the identity
    return x + (_fq_torch(x, axis) - x).detach()


def ste_single_tile_grads(q, k, v, do, causal):
    """float64 autograd of the fake-quant forward with all keys in one tile.

    Q^, K^ (along d), V^ (along the sequence) and P~ (along the keys, per 32) pass gradients
    straight through; the row max is a constant.  With one tile the forward's running max is the
    final row max, so its P~ = MXFP4(exp(s - m)) is exactly the one the backward requantizes.
    Returns O and the gradients of sum(O * dO) with respect to q, k, v.
    """
    tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    B, Hq, N, d = q.shape
    group = Hq // k.shape[1]
    qh = _ste(tq, -1)
    kh = _ste(tk, -1).repeat_interleave(group, dim=1)
    vh = _ste(tv, -2).repeat_interleave(group, dim=1)
    s = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / np.sqrt(d)
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    m = s.max(dim=-1, keepdim=True).values.detach()
    p = torch.exp(s - m)
    pt = _ste(p, -1)
    l = pt.sum(dim=-1, keepdim=True)
    o = torch.matmul(pt, vh) / l
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


STE_CASES = [(False, 1, 1, 64, 64), (False, 2, 2, 128, 128), (True, 2, 2, 256, 64),
             (True, 4, 2, 128, 128), (False, 4, 2, 256, 128), (True, 2, 1, 64, 128)]


@pytest.mark.parametrize("causal,hq,hkv,n,d", STE_CASES)
def test_backward_quantized_equals_ste_autograd(causal, hq, hkv, n, d):
    """Attn-QAT abstract, principles (1) and (2): the backward recomputes the FP4 scores and
    feeds P~ = MXFP4(p)/l to dV, the unquantized P to dS, and the FP4 forward's own O to D.
    With one key tile that is exactly the straight-through gradient of the fake-quant forward."""
    seed = 50 + n + d + 7 * hq + causal
    q, k, v = rand((1, hq, n, d), seed, 2.0), rand((1, hkv, n, d), seed + 1, 1.5), rand((1, hkv, n, d), seed + 2)
    do = rand((1, hq, n, d), seed + 3)
    o, m, l = attn_fwd(q, k, v, causal=causal, bc=n)      # one tile: running max = final max
    ro, gq, gk, gv = ste_single_tile_grads(q, k, v, do, causal)
    assert np.max(np.abs(o - ro)) < 1e-12
    dq, dk, dv = attn_bwd(q, k, v, o, do, m, l, causal=causal, chunk=40)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


def test_ste_pin_rejects_plausible_backward_mistakes():
    """The autograd pin separates the oracle's placement of P~ from three plausible mistakes:
    dV from the unquantized P, dV from MXFP4(P) (quantizing p / l instead of p), and P~/l in dS.
    Each mistake is written out here on one head; each misses the autograd gradient by far more
    than the 1e-12 the oracle meets."""
    n, d = 128, 64
    q, k, v = rand((1, 1, n, d), 90, 2.0), rand((1, 1, n, d), 91, 1.5), rand((1, 1, n, d), 92)
    do = rand((1, 1, n, d), 93)
    o, m, l = attn_fwd(q, k, v, bc=n)
    _, gq, gk, gv = ste_single_tile_grads(q, k, v, do, False)
    qh, kh, vh = fake_quant_mx(q[0, 0], -1), fake_quant_mx(k[0, 0], -1), fake_quant_mx(v[0, 0], 0)
    s = qh @ kh.T / np.sqrt(d)
    p = np.exp(s - m[0, 0][:, None])
    P = p / l[0, 0][:, None]
    Pt = fake_quant_mx(p, -1) / l[0, 0][:, None]
    D = np.sum(do[0, 0] * o[0, 0], axis=1)
    dP = do[0, 0] @ vh.T
    dv_a, dv_b = P.T @ do[0, 0], fake_quant_mx(P, -1).T @ do[0, 0]
    dk_c = (Pt * (dP - D[:, None])).T @ qh / np.sqrt(d)
    dk_ok = (P * (dP - D[:, None])).T @ qh / np.sqrt(d)
    assert np.max(np.abs(dk_ok - gk[0, 0])) < 1e-12          # the oracle's own placement
    assert np.max(np.abs(Pt.T @ do[0, 0] - gv[0, 0])) < 1e-12
    for bad, good in ((dv_a, gv), (dv_b, gv), (dk_c, gk)):
        assert np.max(np.abs(bad - good[0, 0])) > 1e-3
