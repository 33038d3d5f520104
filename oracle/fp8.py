"""FP8 (E4M3) key/value cache -- fp64 oracle.

Test infrastructure only (see ``oracle/__init__.py``).

Source: news article "vLLM, TML Inkling Day-0 support", *Roadmap* (FP8 for
the global-attention layers, which are bound by compute and by the capacity
of the KV cache).  The pages name no format and no scaling, so the readings
here (each listed in the design notes) are:

* the 8-bit format is OCP E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6; codes
  0x7F and 0xFF are NaN; there is no infinity, so the largest finite value is
  1.75 * 2^8 = 448;
* the cache holds code(x / s) with one float scale s for all keys of a layer
  and another for all values; a cached element reads back as value(code) * s;
* encoding rounds to the nearest representable value, ties to the code with
  an even mantissa, and saturates: |x / s| above 448 stores +-448;
* attention over an FP8 cache is the same attention as over a bf16 one, on
  the read-back keys and values (``dequantize``); nothing else changes.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of E4M3 codes (uint8 array or int) as float64; NaN for 0x7F, 0xFF."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# Non-negative finite magnitudes, ascending: code k (k = 0 .. 126) has value
# _MAGS[k] (the encoding is monotone in the low 7 bits).
_MAGS = e4m3_value(np.arange(0x7F))
_VALUES = e4m3_value(np.arange(256))                   # every code, for dequantize


def e4m3_code(x):
    """E4M3 code of float64 values: nearest, ties to even, saturating at 448.
    The sign of a value that rounds to zero is kept (code 0x80 for -0)."""
    x = np.asarray(x, dtype=np.float64)
    assert not np.isnan(x).any()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, len(_MAGS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    k = np.where(pick_hi, hi, lo)
    k = np.where(_MAGS[hi] == a, hi, k)                  # exactly representable
    return (k | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize(x, scale):
    """Codes the cache stores for values x with scale s: code(x / s)."""
    return e4m3_code(np.asarray(x, dtype=np.float64) / float(scale))


def dequantize(code, scale):
    """Values a cache element with these codes reads back as: value * s
    (``e4m3_value`` of each code, looked up from the 256 codes' values)."""
    return _VALUES[np.asarray(code, dtype=np.uint8)] * float(scale)
