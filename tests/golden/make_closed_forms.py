"""Writes closed_forms.json: small cases whose exact results follow by hand
from the definitions on the pages, evaluated here with plain arithmetic.

Nothing here calls the oracle or the HIP library: each expected value is the
closed form stated beside it.  The pages print no worked example, so these
are the stored fixtures the oracle is checked against (tests/test_oracle_golden.py).

Sources (page titles): news article "vLLM, TML Inkling Day-0 support",
Model Architecture / Sconv (window-4 convolution over keys and values),
vLLM Integration & Optimization / Managing the sconv cache (the last three
pre-convolution tokens are kept), Model Architecture / Attention (a learned
relative-position term added to the pre-softmax logits; head size 128).
Readings used where the pages leave a step open: tap 3 multiplies the
current token; the logit is q.k/sqrt(128) + bias[h][min(i-j, R-1)]; a window
W keeps keys with 0 <= i-j <= W-1 (W = 0: full causal).

Run: python tests/golden/make_closed_forms.py
"""
import json
import math
import os

D = 128


def onehot(i, scale=1.0):
    v = [0.0] * D
    v[i] = scale
    return v


cases = []

# ---- sconv: integer taps on an integer ramp with a carried state.
# channel 0 taps (1, 2, 3, 4) over xp = (1, 2, 3, 4, 5):
#   y0 = 1*1 + 2*2 + 3*3 + 4*4 = 30,  y1 = 1*2 + 2*3 + 3*4 + 4*5 = 40
# channel 1 taps (0, 0, 0, 1): the current token passes through.
cases.append({
    "kind": "sconv",
    "cite": "[A] Model Architecture / Sconv; Managing the sconv cache",
    "x": [[4.0, 40.0], [5.0, 50.0]],
    "w": [[1.0, 2.0, 3.0, 4.0], [0.0, 0.0, 0.0, 1.0]],
    "state": [[1.0, 10.0], [2.0, 20.0], [3.0, 30.0]],
    "y": [[30.0, 40.0], [40.0, 50.0]],
    "new_state": [[3.0, 30.0], [4.0, 40.0], [5.0, 50.0]],
})

# ---- attention, q = 0: the weights come from the bias alone.
# Row 1 sees key 0 at distance 1 (bias b1 = 0) and key 1 at distance 0
# (bias b0 = ln 3): weights 1/4 and 3/4, lse = ln(1 + 3) = ln 4.
# Row 0 sees only key 0 at distance 0: o = v0, lse = ln 3.
b0, b1 = math.log(3.0), 0.0
v0, v1 = onehot(0), onehot(1, 2.0)
cases.append({
    "kind": "attention",
    "cite": "[A] Model Architecture / Attention (relative term added to the logits)",
    "window": 0,
    "q": [[onehot(0, 0.0)], [onehot(0, 0.0)]],
    "k": [[onehot(2)], [onehot(3)]],
    "v": [[v0], [v1]],
    "bias": [[b0, b1]],
    "out": [[v0], [[0.25 * a + 0.75 * b for a, b in zip(v0, v1)]]],
    "lse": [[math.log(3.0)], [math.log(4.0)]],
})

# ---- attention, the 1/sqrt(128) scale: q = sqrt(128) ln 2 e0 against
# k0 = e0 (logit ln 2) and k1 = e1 (logit 0), zero bias: row 1 weights 2/3
# on key 0 and 1/3 on key 1; lse = ln(2 + 1) = ln 3.
a = math.sqrt(D) * math.log(2.0)
u0, u1 = onehot(5, 3.0), onehot(6, -1.5)
cases.append({
    "kind": "attention",
    "cite": "[A] Model Architecture / Attention (head size 128)",
    "window": 0,
    "q": [[onehot(0, a)], [onehot(0, a)]],
    "k": [[onehot(0)], [onehot(1)]],
    "v": [[u0], [u1]],
    "bias": [[0.0, 0.0]],
    "out": [[u0], [[(2.0 * x + y) / 3.0 for x, y in zip(u0, u1)]]],
    "lse": [[math.log(2.0)], [math.log(3.0)]],
})

# ---- attention, window 2 and a one-entry table (every distance takes
# bias[0]): row 2 sees keys 1 and 2 only, with equal logits (q = 0), so
# o = (v1 + v2) / 2 and lse = c + ln 2 for the constant bias c = 0.5.
w0, w1, w2 = onehot(7, 9.0), onehot(8, 1.0), onehot(9, 3.0)
cases.append({
    "kind": "attention",
    "cite": "[A] Model Architecture / Attention (sliding-window layers)",
    "window": 2,
    "q": [[onehot(0, 0.0)]] * 3,
    "k": [[onehot(1)], [onehot(2)], [onehot(3)]],
    "v": [[w0], [w1], [w2]],
    "bias": [[0.5]],
    "out": [[w0], [[(x + y) / 2.0 for x, y in zip(w0, w1)]],
            [[(x + y) / 2.0 for x, y in zip(w1, w2)]]],
    "lse": [[0.5], [0.5 + math.log(2.0)], [0.5 + math.log(2.0)]],
})

path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
with open(path, "w") as f:
    json.dump({"note": "closed-form cases written by make_closed_forms.py; see its header",
               "cases": cases}, f)
print("wrote", path)
