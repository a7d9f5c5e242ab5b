"""bfloat16 <-> float64 codec (test infrastructure only).

The KV cache and the activations of the decode path are bfloat16 (the pages
benchmark a bf16-KV engine; the fused prologue writes bf16 q/gate/K/V).  A
bfloat16 value is the upper 16 bits of an IEEE binary32 value, so decoding is
exact; encoding rounds to nearest, ties to even (the IEEE default, and the
rounding the GPU's bf16 stores use).

The encoder rounds the float64 value *directly* to bf16 (no detour through
binary32, which could round twice).
"""

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_MIN_QUANTUM_EXP = -133  # smallest bf16 subnormal is 2**-126 * 2**-7


def to_f64(bits):
    """Decode bf16 bit patterns (uint16/int16 array) to float64, exactly."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def from_f64(x):
    """Round float64 values to bf16 bit patterns (uint16), nearest-even.

    For finite x the bf16 grid spacing near |x| is 2**(e-8) where
    x = m * 2**e with 0.5 <= |m| < 1 (8 significant bits), floored at the
    subnormal spacing 2**-133.  x / spacing is rounded with numpy's
    half-to-even ``rint`` and scaled back; the result is exactly a bf16 value
    (hence also a binary32 value), whose upper 16 bits are the encoding.
    Values beyond the largest finite bf16 after rounding become +-inf; NaN
    stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)
    qexp = np.maximum(e.astype(np.int64) - 8, _MIN_QUANTUM_EXP)
    y = np.ldexp(np.rint(np.ldexp(xf, -qexp)), qexp)
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, y), y)
    out[finite] = y
    out[~finite] = x[~finite]
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def round_f64(x):
    """float64 -> nearest bf16 value, returned as float64."""
    return to_f64(from_f64(x))


def ulp(x):
    """Spacing of the bf16 grid at |x| (the ulp used by tolerance checks)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x == 0, 1.0, x))
    sp = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 8, _MIN_QUANTUM_EXP))
    return np.where(x == 0, np.ldexp(1.0, _MIN_QUANTUM_EXP), sp)
