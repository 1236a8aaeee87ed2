"""Rounding onto the bfloat16 grid, computed in float64.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module.

The pages fix bf16 as the storage type of activations: the per-token
all-reduce payload of Llama-3.1-8B is hidden 4096 x 2 B = 8 KiB ("张量、流水线与
数据并行", section 每 token 的通信量), and that page's whole traffic estimate
assumes two-byte activations. They do not name a rounding mode; the oracle takes
IEEE round to nearest, ties to even, the binary default.

bfloat16 is binary32 with the fraction cut to 7 stored bits: same exponent
range (normal exponents -126..127), 8 significant bits, gradual underflow down
to 2**-133, overflow to infinity at and above 2**128 - 2**119 after rounding.

The rounding is done arithmetically, not by bit manipulation: the value is
split into significand and exponent with ``frexp`` (exact), scaled so that one
unit in the last bf16 place becomes 1, rounded with ``rint`` (ties to even),
and scaled back. Every step is exact in float64 for any finite input.
"""

import numpy as np

_FRACTION_BITS = 7          # stored fraction bits of bfloat16
_MIN_NORMAL_EXP = -126      # exponent of the smallest normal number
_OVERFLOW = 2.0 ** 128      # rounded magnitudes at or above this are infinite


def round_bf16(x):
    """Return the bf16 value nearest to each element of ``x`` (ties to even),
    as a float64 array.

    NaN stays NaN, infinities and signed zeros keep their sign, values that
    round beyond the largest finite bf16 become infinite.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    sel = np.isfinite(x) & (x != 0.0)
    v = x[sel]
    # v = m * 2**e with 0.5 <= |m| < 1, so the leading bit has weight 2**(e-1).
    _, e = np.frexp(v)
    lead = np.maximum(e - 1, _MIN_NORMAL_EXP)      # subnormals share the min exponent
    ulp_exp = lead - _FRACTION_BITS
    q = np.ldexp(v, -ulp_exp)                      # exact: power-of-two scaling
    r = np.ldexp(np.rint(q), ulp_exp)              # rint rounds half to even
    r = np.where(np.abs(r) >= _OVERFLOW, np.copysign(np.inf, v), r)
    out[sel] = r
    return out


def bf16_bits(x):
    """Bit pattern (uint16) of the bf16 values in ``x``, which must already be
    on the bf16 grid. Used only to compare signed zeros and payloads exactly."""
    x = np.asarray(x, dtype=np.float64)
    if not np.array_equal(round_bf16(x), x, equal_nan=True):
        raise ValueError("bf16_bits: value not representable in bfloat16")
    f32 = x.astype(np.float32)                     # exact: bf16 is a subset of binary32
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
