"""EFQ-Softmax probability codes (exp-free), float64 CPU oracle -- a reading.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (EFQ-Softmax abstract, on the AVQ Attention page and the
theflow "related" summary): the probability operand of PV is block-scaled
E2M1; per microscaling block an exponent-only scale is chosen from the local
maximum; the shifted scores are mapped to a normalised residual domain, and
the non-negative E2M1 codes come from a single affine rule, without
evaluating the exponential first.  The same operand feeds the numerator and
the denominator updates.

What they leave open, and the reading taken here:

* the scale is the MX exponent of the block's largest probability, as for
  exp-then-quantize: e = clamp(floor(x_max) - 2, -127, 127) with x = log2 p
  = (s - m) / ln 2 the shifted score in base 2 (x_max < -126 counts as -127);
* the normalised residual is y = x - e, the base-2 logarithm of p / 2^e;
* the affine rule is k = clamp(round_half_even(A y + B), 0, 7), with A, B the
  least-squares line through the points (log2 v_k, k) of the seven non-zero
  E2M1 magnitudes v_k = 0.5, 1, 1.5, 2, 3, 4, 6 (k = 1..7): the code index is
  read as an affine function of log2 of the value it stands for (exactly so,
  A = 2 and B = 2, for the powers of two; the fit also places the 1.5 * 2^j
  codes and the 0.5 code).  A = 1.7470566..., B = 2.3141184...;
* the operand value is the code's E2M1 magnitude times 2^e.

The rule differs from exp-then-quantize by at most one code step (a test pins
this) and gives the block maximum of a block whose largest probability is a
power of two the same code as exp-then-quantize.

Parity status: the rule itself is this reading (the pages state no formula),
so GPU-versus-oracle parity for this mode checks the implementation of the
reading, not the pages' exact numbers.  Pins (tests/test_oracle_efq.py):
the fitted line against its closed form, integer points of A y + B map to that
code and half-way points to the even neighbour, codes are monotone in x and
within one step of exp-then-quantize, a block max of p = 2^j gives P~ = p,
masked blocks give 0, Q = 0 gives the mean of V^ (causal: prefix mean).
"""

import numpy as np

from .mx import E2M1_GRID, MX_BLOCK

# least-squares line k ~ A log2(v_k) + B over the non-zero E2M1 magnitudes (a library fit)
EFQ_A, EFQ_B = np.polyfit(np.log2(E2M1_GRID[1:]), np.arange(1, 8, dtype=np.float64), 1)


def efq_block_exponent(x_max):
    """MX exponent of a block whose largest probability is 2^x_max (x_max may be -inf)."""
    x_max = np.asarray(x_max, dtype=np.float64)
    ex = np.where(x_max >= -126.0, np.floor(np.where(np.isfinite(x_max), x_max, 0.0)), -127.0)
    return np.clip(ex - 2.0, -127.0, 127.0)


def efq_codes(x, axis=-1):
    """EFQ codes (0..7) and block exponents for base-2 log-probabilities x (<= 0, -inf allowed).

    Blocks of 32 along `axis`.  Returns (codes int64 same shape as x, e with the block axis
    reduced).
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("length along the axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    e = efq_block_exponent(xb.max(axis=-1))
    y = xb - e[..., None]
    t = np.where(np.isneginf(y), -1.0, EFQ_A * y + EFQ_B)
    k = np.clip(np.round(t), 0, 7).astype(np.int64)      # np.round: half to even
    return np.moveaxis(k.reshape(x.shape), -1, axis), e


def efq_fake_quant(x, axis=-1):
    """The EFQ operand values E2M1[k] * 2^e for base-2 log-probabilities x, blocks along axis."""
    k, e = efq_codes(x, axis=axis)
    k = np.moveaxis(k, axis, -1)
    n = k.shape[-1]
    vals = E2M1_GRID[k].reshape(k.shape[:-1] + (n // MX_BLOCK, MX_BLOCK)) * np.exp2(e)[..., None]
    return np.moveaxis(vals.reshape(k.shape), -1, axis)
