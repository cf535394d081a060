"""Oracle's own bfloat16 rounding (test infrastructure; see package docstring).

bfloat16 keeps the float32 exponent and 7 explicit mantissa bits.  Rounding is
to the nearest representable value, ties to the even mantissa.  Written here
from that definition on float64 bit patterns (52 mantissa bits -> keep 7, drop
45), so a single rounding from the exact fp64 value.  Valid for zeros and for
magnitudes in bfloat16's normal range (2**-126 .. ~3.4e38), which covers every
value the decoder produces; inf/nan pass through unchanged.
"""

from __future__ import annotations

import numpy as np

_DROP = 45  # 52 - 7 mantissa bits discarded
_LOW_MASK = np.uint64((1 << _DROP) - 1)
_HALF_MINUS_ONE = np.uint64((1 << (_DROP - 1)) - 1)


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each element, returned as float64."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(_DROP)) & np.uint64(1)
    rounded = (bits + _HALF_MINUS_ONE + lsb) & ~_LOW_MASK
    out = rounded.view(np.float64).copy()
    special = ~np.isfinite(a)
    if special.any():
        out[special] = a[special]
    return out
