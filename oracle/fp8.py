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

For FP8 matrix products in the attention itself (the same *Roadmap* item:
the global layers are bound by compute as well), the queries and the softmax
probabilities are rounded to E4M3 too.  The pages give no scheme; the one
used here (listed in the design notes) is

* queries: one scale per tile of 256 consecutive query rows of a sequence's
  chunk (rows 256t .. 256t+255) and one query head.  With amax the largest
  |q| of the tile, the codes are code(fp32(q) * fp32(448 / amax)) (both
  operations in float32, as the kernel computes them) and the read-back
  value is value(code) * fp32(amax / 448); an all-zero tile reads back as
  zeros (``quantize_query_tiles``);
* probabilities: rounded to the nearest E4M3 value (ties to even), with the
  softmax's row sum taken over the rounded values.  This rounding happens
  inside the online softmax, on values whose scale depends on the kernel's
  running maximum, so it is not reproduced here; ``e4m3_spacing`` gives the
  size of the rounding step that the tests' error bounds are built from.
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


def e4m3_spacing(x):
    """Distance between consecutive E4M3 values around |x| (|x| <= 448): 2^-9
    below the smallest normal 2^-6, else 2^(floor(log2 |x|) - 3)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3.0))


def quantize_query_tiles(q, cu_seqlens, tile=256):
    """Read-back values of queries rounded to E4M3 with one scale per tile of
    ``tile`` rows of each sequence's chunk and per query head.

    q : [num_tokens, Hq, d] (float32-representable values); cu_seqlens :
    [num_seqs + 1].  Returns (q_read_back float64 [num_tokens, Hq, d],
    codes uint8 [num_tokens, Hq, d])."""
    q32 = np.asarray(q, dtype=np.float32)
    out = np.zeros(q32.shape, dtype=np.float64)
    codes = np.zeros(q32.shape, dtype=np.uint8)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        for r0 in range(int(cu[b]), int(cu[b + 1]), tile):
            r1 = min(r0 + tile, int(cu[b + 1]))
            for h in range(q32.shape[1]):
                x = q32[r0:r1, h, :]
                amax = np.float32(np.abs(x).max())
                if amax == 0.0:
                    continue                      # codes 0, values 0
                inv = np.float32(np.float32(E4M3_MAX) / amax)
                c = e4m3_code((x * inv).astype(np.float32).astype(np.float64))
                codes[r0:r1, h, :] = c
                out[r0:r1, h, :] = _VALUES[c] * float(np.float32(amax / np.float32(E4M3_MAX)))
    return out, codes
