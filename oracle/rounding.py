"""Storage rounding for the oracle (test infrastructure only).

The oracle computes in float64 and rounds to the workload's storage dtype at
the points where the GPU path writes a tensor to memory (layer input, Q/K/V,
attention output, x after each residual, normed activations, the FFN
intermediate, logits).  The pages fix no precision; this follows the storage
precision of each workload.

  "f64":  no rounding (used by pins against float64 library routines)
  "f32":  IEEE binary32, round to nearest even (NumPy's float32 cast)
  "bf16": bfloat16 (8 significant bits), round to nearest even, computed here
          directly from the float64 value (no detour through float32)
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_STEP = 2.0 ** -133


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 entry (ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x)
    xf = x[finite]
    mag = np.abs(xf)
    res = np.empty_like(xf)
    normal = mag >= _BF16_MIN_NORMAL
    # Normal range: x = m * 2**e with 0.5 <= |m| < 1; keep 8 significant bits.
    m, e = np.frexp(xf[normal])
    res[normal] = np.ldexp(np.rint(m * 256.0), e - 8)     # np.rint rounds half to even
    # Subnormal range: fixed spacing 2**-133.
    sub = ~normal
    res[sub] = np.rint(xf[sub] / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP
    # Values that round past the largest finite bfloat16 overflow to infinity.
    over = np.abs(res) > _BF16_MAX
    res[over] = np.copysign(np.inf, res[over])
    out[finite] = res
    return out


def to_storage(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")
