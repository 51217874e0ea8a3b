"""Correctly rounded conversion from fp64 and ulp distances (test infrastructure).

Round-to-nearest, ties-to-even, directly from float64 to a binary format with
``p`` significand bits (implicit bit included) and minimum normal exponent
``emin``: the value is scaled by a power of two so that its last kept bit is
the units digit, rounded with ``np.rint`` (ties to even) and scaled back. All
three steps are exact in float64, so there is no double rounding (converting
float64 -> float32 -> bfloat16 in two steps can round twice). Results above
the largest finite value become +-inf; subnormals keep the fixed quantum
2**(emin - p + 1).
"""

import numpy as np

FORMATS = {
    # name: (significand bits incl. implicit, emin, emax)
    "bf16": (8, -126, 127),
    "fp16": (11, -14, 15),
    "fp32": (24, -126, 127),
}


def round_to(x, fmt):
    """Round float64 values to the nearest value of ``fmt`` (RNE); returns float64."""
    p, emin, emax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)                      # |x| = m * 2**e2, m in [0.5, 1)
    q = np.maximum(e2 - 1, emin) - (p - 1)    # exponent of the last kept bit
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    big = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    y = np.where(np.abs(y) > big, np.copysign(np.inf, y), y)
    out[fin] = y
    return out


def _bits(v, fmt):
    v = np.asarray(v)
    if fmt == "fp16":
        return v.astype(np.float16).view(np.uint16).astype(np.int64), 16
    if fmt == "fp32":
        return v.astype(np.float32).view(np.uint32).astype(np.int64), 32
    if fmt == "bf16":
        b = v.astype(np.float32).view(np.uint32).astype(np.int64)
        return b >> 16, 16
    raise ValueError(fmt)


def ordered_int(v, fmt):
    """Map values representable in ``fmt`` to integers whose order and
    differences follow the format's ordering; +0 and -0 both map to 0."""
    b, w = _bits(v, fmt)
    sign = (b >> (w - 1)) & 1
    mag = b & ((1 << (w - 1)) - 1)
    return np.where(sign == 1, -mag, mag)


def ulp_distance(a, b, fmt):
    """Number of representable ``fmt`` values between a and b (elementwise)."""
    return np.abs(ordered_int(a, fmt) - ordered_int(b, fmt))
