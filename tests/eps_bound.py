"""The smallest softening the entry points admit: the target's own term is
m * 0 * eps^-3 (d = 0), and it is +0 only while eps^-3, evaluated as the term
evaluates it in float32, is finite. Computed here with NumPy float32
arithmetic (every operation rounded to float32), independently of the library
and of the oracle."""

import numpy as np


def self_term_finite(eps: float) -> bool:
    e = np.float32(eps)
    e2 = np.float32(e * e)
    if not (np.isfinite(e) and e2 > 0):
        return False
    inv = np.float32(np.float32(1.0) / np.sqrt(e2))
    with np.errstate(over="ignore"):  # the overflow is what is being detected
        return bool(np.isfinite(np.float32(np.float32(inv * inv) * inv)))


def _f32(bits: int) -> float:
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def smallest_eps():
    """(smallest admissible float32 eps, the float32 just below it), by
    bisection over the ordered bit patterns of positive floats."""
    a, z = int(np.float32(1e-13).view(np.uint32)), int(np.float32(1e-12).view(np.uint32))
    assert not self_term_finite(_f32(a)) and self_term_finite(_f32(z))
    while z - a > 1:
        m = (a + z) // 2
        a, z = (a, m) if self_term_finite(_f32(m)) else (m, z)
    return _f32(z), _f32(a)
