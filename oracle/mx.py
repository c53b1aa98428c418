"""MXFP4 (block-scaled E2M1) quantizer, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: operands are block-scaled E2M1 values that share an
exponent-only scale per microscaling block (EFQ-Softmax abstract; the
SageAttention3 "Microscaling FP4" title on the Pengle Zhang author page).
What they leave open, and the reading taken here (the OCP Microscaling v1.0
MXFP4 format that the name "MXFP4" refers to):

* block = 32 contiguous elements along the contraction axis, starting at
  index 0 of that axis;
* E2M1 element: sign bit (bit 3) + 2 exponent bits + 1 mantissa bit, the
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no Inf, no NaN;
* E8M0 scale byte = e + 127 with e = floor(log2(amax)) - 2, where 2 is the
  exponent of the largest E2M1 magnitude (6 = 1.5 * 2^2); amax below the
  smallest fp32 normal (2^-126) counts as e_x = -127; e is clamped to
  [-127, 127] so the byte 0xFF (NaN) is never produced;
* element code = round-to-nearest-even of x / 2^e onto the grid, ties to the
  even mantissa bit, saturating at 6; the sign is kept, also for values that
  round to zero (-0 -> code 0x8).

Parity pins (tests/test_oracle_mx.py): the 16-code decode table against the
grid; the element rule against two independent formulations (brute-force
argmin over the grid with the tie rule, and numpy's banker's rounding on a
rescaled mantissa) over every finite bfloat16 value; the scale rule against
its closed form; identity on representable blocks; sign and power-of-two
equivariance; idempotence.
"""

import numpy as np

MX_BLOCK = 32

# Magnitudes of the eight non-negative E2M1 codes 0..7 (sign is bit 3).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# Largest E2M1 exponent (6 = 1.5 * 2**2).
_E2M1_EMAX = 2


def decode_e2m1(codes):
    """Value of each 4-bit E2M1 code (int array, 0..15) as float64."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_GRID[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


def e2m1_round_codes(v):
    """Round float64 values ``v`` (already divided by the block scale) to E2M1.

    Round-to-nearest-even onto the grid, saturating at 6, sign kept.  Written
    as the interval table of that rounding: a value exactly halfway between
    two grid points goes to the code whose mantissa bit is 0 (the even code),
    so 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    mag = ((a > 0.25).astype(np.int64)
           + (a >= 0.75)
           + (a > 1.25)
           + (a >= 1.75)
           + (a > 2.5)
           + (a >= 3.5)
           + (a > 5.0))
    sign = np.signbit(v).astype(np.int64) << 3
    return (mag | sign).astype(np.uint8)


def mx_scale_exponent(amax):
    """Shared exponent e of a block from its max magnitude (float64 array).

    e = clamp(floor(log2 amax) - 2, -127, 127); amax < 2**-126 (including
    0) is treated as floor(log2 amax) = -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    small = amax < 2.0 ** -126
    # np.frexp: amax = f * 2**k with f in [0.5, 1) -> floor(log2 amax) = k - 1 exactly.
    _, k = np.frexp(np.where(small, 1.0, amax))
    ex = np.where(small, -127, k.astype(np.int64) - 1)
    return np.clip(ex - _E2M1_EMAX, -127, 127).astype(np.int64)


def quantize_mx(x, axis=-1):
    """MXFP4-quantize ``x`` along ``axis`` (length a multiple of 32).

    Returns ``(codes, scales)``: ``codes`` uint8 (one 4-bit code per element,
    unpacked, same shape as x), ``scales`` uint8 E8M0 bytes with the axis
    length divided by 32.
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("quantized axis length %d is not a multiple of %d" % (n, MX_BLOCK))
    xb = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    e = mx_scale_exponent(amax)
    v = xb / np.ldexp(1.0, e)[..., None]          # exact: division by a power of two
    codes = e2m1_round_codes(v).reshape(x.shape)
    scales = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize_mx(codes, scales, axis=-1):
    """Inverse of the representation: value = decode(code) * 2**(scale-127)."""
    codes = np.moveaxis(np.asarray(codes), axis, -1)
    scales = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64)
    vals = decode_e2m1(codes)
    n = vals.shape[-1]
    vb = vals.reshape(vals.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    out = vb * np.ldexp(1.0, scales - 127)[..., None]
    return np.moveaxis(out.reshape(vals.shape), -1, axis)


def fake_quant_mx(x, axis=-1):
    """Quantize then dequantize along ``axis`` (float64 in, float64 out)."""
    c, s = quantize_mx(x, axis)
    return dequantize_mx(c, s, axis)


def pack_nibbles(codes, axis=-1):
    """Two codes per byte along ``axis``: element 2c -> bits 3..0, 2c+1 -> bits 7..4."""
    c = np.moveaxis(np.asarray(codes, dtype=np.uint8), axis, -1)
    packed = (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)
    return np.moveaxis(packed.astype(np.uint8), -1, axis)


def unpack_nibbles(packed, axis=-1):
    """Inverse of :func:`pack_nibbles`."""
    p = np.moveaxis(np.asarray(packed, dtype=np.uint8), axis, -1)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return np.moveaxis(out, -1, axis)
