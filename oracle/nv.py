"""NVFP4-style operands (E2M1, 16-element blocks, E4M3 block scale, fp32 tensor scale), CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: only the name.  NVFP4 appears as a 4-bit format for
linear layers (TetraJet-v2 abstract) and beside MXFP4 and HiF4 among the
4-bit formats that are compared (RFQ abstract; HiFA4 abstract for HIF4).  No
page gives a block size, a scale type or a rounding rule.  The reading taken
here is the published NVFP4 layout the name refers to, with every open
rounding step fixed so that a decision is taken in fp32, the precision the
GPU path computes in:

* element: E2M1 code as for MXFP4 (sign bit 3, magnitudes
  {0, .5, 1, 1.5, 2, 3, 4, 6}, round half to even, saturate at 6);
* block: 16 contiguous elements along the contraction axis, from index 0;
* block scale: an unsigned FP8 E4M3 byte (4 exponent bits, bias 7, 3
  mantissa bits, subnormals; largest value 448, the NaN byte 0x7F never
  written), value S;
* tensor scale: one fp32 G per quantized tensor (all of Q, all of K, all of
  V): G = max(amax / 2688, 2^-117) in fp32, 2688 = 6 * 448 so that the
  tensor's largest block gets S = 448; the floor keeps S * G a normal fp32
  number for every non-zero S;
* per block, in fp32 with round-to-nearest-even after each operation:
  D = 6 * G; s = amax_block / D; S = E4M3 round-to-nearest-even of s (ties to
  the even mantissa, saturating at 448); sigma = S * G; v = x / sigma;
  code = E2M1 rounding of v.  A block with S = 0 gets the zero code with the
  element's sign;
* value = G * S * E2M1(code).

The probability operand P~ of the PV product is quantized with the same
format per 16 keys.  Since 0 <= p <= 1 and the row maximum has p = 1, its
tensor scale is the one the recipe gives for amax = 1: G_P = 1/2688.  Per
block: S = E4M3(max p * 448), value = E2M1(p * 2688 / S) * S / 2688 (0 when
S = 0).  The row maximum then has P~ = 1 exactly.  P~ is not an output, so it
is evaluated in float64 here.

Parity pins (tests/test_oracle_nv.py): the E4M3 decode table against its
bit-field definition and hand values; E4M3 rounding against an independent
quantum-and-banker's-rounding formulation and brute-force nearest over the
table; identity on blocks that are exactly representable; power-of-two
equivariance of codes and scales; the tensor's largest element getting the
code of 6 and S = 448; the error bound of each element; P~ = 1 at the row
maximum; Q = 0 giving the mean of V^ in the forward.
"""

import numpy as np

from .mx import E2M1_GRID, e2m1_round_codes

NV_BLOCK = 16
E4M3_MAX = 448.0
NV_TENSOR_DIV = 2688.0          # 6 * 448: E2M1 max times E4M3 max
NV_G_MIN = 2.0 ** -117          # floor of G: S * G stays a normal fp32 for S >= 2^-9


def decode_e4m3(b):
    """Value of each FP8 E4M3 byte (bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa)."""
    b = np.asarray(b).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, np.maximum(e, 1) - 10))
    return np.where((b & 0x80) != 0, -mag, mag)


# the 127 non-negative finite E4M3 values, codes 0x00..0x7E, in ascending order
E4M3_POS = decode_e4m3(np.arange(127))


def e4m3_round_codes(t):
    """E4M3 byte nearest to each t >= 0 (float64); a tie goes to the even code; saturates at 448."""
    t = np.asarray(t, dtype=np.float64)
    hi = np.clip(np.searchsorted(E4M3_POS, t, side="left"), 1, 126)
    lo = hi - 1
    d_lo = t - E4M3_POS[lo]
    d_hi = E4M3_POS[hi] - t
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8)


def nv_tensor_scale(x):
    """(G, amax) of a tensor: amax = max |x| (exact), G = max(fp32(amax / 2688), 2^-117), both fp32."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else np.float32(0)
    g = np.float32(amax) / np.float32(NV_TENSOR_DIV)
    return np.float32(max(g, np.float32(NV_G_MIN))), amax


def quantize_nv(x, axis=-1, g=None):
    """NVFP4-quantize ``x`` along ``axis`` (length a multiple of 16) with tensor scale ``g``.

    ``g`` defaults to the scale of ``x`` itself; pass the whole tensor's scale when ``x`` is a
    slice of it.  Returns ``(codes, scales, g)``: codes uint8 (one 4-bit code per element, same
    shape as x), scales uint8 E4M3 bytes with the axis length divided by 16, g float32.
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % NV_BLOCK:
        raise ValueError("quantized axis length %d is not a multiple of %d" % (n, NV_BLOCK))
    g = nv_tensor_scale(x)[0] if g is None else np.float32(g)
    xb = x.reshape(x.shape[:-1] + (n // NV_BLOCK, NV_BLOCK))
    d6 = np.float32(6.0) * g                                         # fp32
    amax = np.max(np.abs(xb), axis=-1).astype(np.float32)            # exact (bf16 inputs)
    s = amax / d6                                                    # fp32 division
    S = e4m3_round_codes(s.astype(np.float64))
    sigma = decode_e4m3(S).astype(np.float32) * g                    # fp32
    with np.errstate(divide="ignore", invalid="ignore"):
        v = xb.astype(np.float32) / sigma[..., None]                # fp32 division
    codes = e2m1_round_codes(np.where(S[..., None] == 0, 0.0, v.astype(np.float64)))
    codes = np.where(S[..., None] == 0, np.signbit(xb).astype(np.uint8) << 3, codes).astype(np.uint8)
    return np.moveaxis(codes.reshape(x.shape), -1, axis), np.moveaxis(S, -1, axis), g


def dequantize_nv(codes, scales, g, axis=-1):
    """value = G * S * E2M1(code), float64."""
    codes = np.moveaxis(np.asarray(codes).astype(np.int64), axis, -1)
    S = decode_e4m3(np.moveaxis(np.asarray(scales), axis, -1))
    mag = E2M1_GRID[codes & 7]
    vals = np.where((codes & 8) != 0, -mag, mag)
    n = vals.shape[-1]
    vb = vals.reshape(vals.shape[:-1] + (n // NV_BLOCK, NV_BLOCK))
    out = vb * S[..., None] * np.float64(g)
    return np.moveaxis(out.reshape(vals.shape), -1, axis)


def fake_quant_nv(x, axis=-1, g=None):
    """Quantize then dequantize along ``axis`` with tensor scale ``g`` (float64 out)."""
    c, s, g = quantize_nv(x, axis, g)
    return dequantize_nv(c, s, g, axis)


def nv_p_fake_quant(p, axis=-1):
    """P~ of probabilities 0 <= p <= 1 per 16 along ``axis``, tensor scale 1/2688 (float64)."""
    p = np.moveaxis(np.asarray(p, dtype=np.float64), axis, -1)
    n = p.shape[-1]
    if n % NV_BLOCK:
        raise ValueError("axis length %d is not a multiple of %d" % (n, NV_BLOCK))
    pb = p.reshape(p.shape[:-1] + (n // NV_BLOCK, NV_BLOCK))
    S = decode_e4m3(e4m3_round_codes(pb.max(axis=-1) * E4M3_MAX))[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(S > 0, pb * NV_TENSOR_DIV / S, 0.0)
    out = E2M1_GRID[e2m1_round_codes(v) & 7] * S / NV_TENSOR_DIV
    return np.moveaxis(out.reshape(p.shape), -1, axis)
