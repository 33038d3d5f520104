"""Pins of the sconv oracle against things other than itself.

The pages print no worked example for the short convolution, so the oracle is
pinned by (a) the identity it must reduce to with delta taps, (b) torch's
float64 depthwise ``conv1d`` with causal left padding (a library routine), (c)
a closed form on a ramp input, (d) chunking / state-carry consistency, which
is what the three-token cache exists for, and (e) linearity.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_delta_current_tap_is_identity():
    # Taps (0, 0, 0, 1): tap 3 weights the current token, so y == x.
    x = _rand(37, 16)
    w = np.zeros((16, 4)); w[:, 3] = 1.0
    y, st = oracle.sconv_sequence(x, w, _rand(3, 16, seed=1))
    np.testing.assert_array_equal(y, x)
    np.testing.assert_array_equal(st, x[-3:])


@pytest.mark.parametrize("tap", [0, 1, 2])
def test_delta_older_tap_is_shift_through_state(tap):
    # Tap k alone delays the signal by 3 - k tokens; the first 3 - k outputs
    # come from the cached state.
    x = _rand(20, 8)
    state = _rand(3, 8, seed=2)
    w = np.zeros((8, 4)); w[:, tap] = 1.0
    y, _ = oracle.sconv_sequence(x, w, state)
    lag = 3 - tap
    full = np.concatenate([state, x])
    np.testing.assert_array_equal(y, full[3 - lag:3 - lag + 20])


def test_matches_torch_conv1d_fresh_state():
    x = _rand(50, 12)
    w = _rand(12, 4, seed=3)
    y, _ = oracle.sconv_sequence(x, w, None)
    xt = torch.from_numpy(x.T.copy())[None]              # [1, C, n]
    wt = torch.from_numpy(w.copy())[:, None, :]          # [C, 1, 4]
    ref = F.conv1d(F.pad(xt, (3, 0)), wt, groups=12)[0].T.numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


def test_matches_torch_conv1d_with_state():
    x = _rand(9, 6)
    state = _rand(3, 6, seed=4)
    w = _rand(6, 4, seed=5)
    y, _ = oracle.sconv_sequence(x, w, state)
    xt = torch.from_numpy(np.concatenate([state, x]).T.copy())[None]
    ref = F.conv1d(xt, torch.from_numpy(w.copy())[:, None, :], groups=6)[0].T
    np.testing.assert_allclose(y, ref.numpy(), rtol=0, atol=1e-13)


def test_ramp_closed_form():
    # x[t] = t on every channel, fresh (zero) state:
    # y[t] = a (t-3) + b (t-2) + c (t-1) + d t for t >= 3.
    n = 12
    x = np.tile(np.arange(n, dtype=np.float64)[:, None], (1, 3))
    a, b, c, d = 0.5, -1.25, 2.0, 0.75
    w = np.tile(np.array([[a, b, c, d]]), (3, 1))
    y, st = oracle.sconv_sequence(x, w)
    t = np.arange(3, n)
    expect = a * (t - 3) + b * (t - 2) + c * (t - 1) + d * t
    np.testing.assert_allclose(y[3:, 0], expect, atol=1e-14)
    # early outputs only see the zero state on the left
    assert y[0, 0] == 0.0
    assert y[1, 0] == pytest.approx(d * 1)
    assert y[2, 0] == pytest.approx(c * 1 + d * 2)
    np.testing.assert_array_equal(st[:, 0], [n - 3, n - 2, n - 1])


@pytest.mark.parametrize("cuts", [[1], [2], [3], [1, 2], [5, 6, 7], [1, 1, 1, 1], [10]])
def test_chunked_with_carried_state_equals_whole(cuts):
    x = _rand(24, 10, seed=6)
    w = _rand(10, 4, seed=7)
    s0 = _rand(3, 10, seed=8)
    y_full, st_full = oracle.sconv_sequence(x, w, s0)
    ys, st, t = [], s0, 0
    for c in cuts + [24 - sum(cuts)]:
        y, st = oracle.sconv_sequence(x[t:t + c], w, st)
        ys.append(y)
        t += c
    np.testing.assert_allclose(np.concatenate(ys), y_full, atol=1e-14)
    np.testing.assert_array_equal(st, st_full)


def test_short_chunk_state_keeps_old_rows():
    s0 = _rand(3, 4, seed=9)
    x = _rand(2, 4, seed=10)
    _, st = oracle.sconv_sequence(x, np.ones((4, 4)), s0)
    np.testing.assert_array_equal(st, np.concatenate([s0[2:], x]))
    _, st0 = oracle.sconv_sequence(x[:0], np.ones((4, 4)), s0)
    np.testing.assert_array_equal(st0, s0)


def test_linearity():
    x1, x2 = _rand(15, 5, seed=11), _rand(15, 5, seed=12)
    w1, w2 = _rand(5, 4, seed=13), _rand(5, 4, seed=14)
    a, b = 1.7, -0.3
    y12, _ = oracle.sconv_sequence(a * x1 + b * x2, w1)
    y1, _ = oracle.sconv_sequence(x1, w1)
    y2, _ = oracle.sconv_sequence(x2, w1)
    np.testing.assert_allclose(y12, a * y1 + b * y2, atol=1e-13)
    yw, _ = oracle.sconv_sequence(x1, a * w1 + b * w2)
    yw2, _ = oracle.sconv_sequence(x1, w2)
    np.testing.assert_allclose(yw, a * y1 + b * yw2, atol=1e-13)


def test_batch_routes_states_and_offsets():
    rng = np.random.default_rng(15)
    C = 8
    lens = [5, 1, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = rng.standard_normal((cu[-1], C))
    v = rng.standard_normal((cu[-1], C))
    w = rng.standard_normal((2, C, 4))
    state = rng.standard_normal((6, 2, 3, C))
    slots = np.array([4, 0, 2, 5])
    ko, vo, ns = oracle.sconv_batch(k, v, w, state, slots, cu)
    for b, s in enumerate(slots):
        yk, sk = oracle.sconv_sequence(k[cu[b]:cu[b + 1]], w[0], state[s, 0])
        yv, sv = oracle.sconv_sequence(v[cu[b]:cu[b + 1]], w[1], state[s, 1])
        np.testing.assert_array_equal(ko[cu[b]:cu[b + 1]], yk)
        np.testing.assert_array_equal(vo[cu[b]:cu[b + 1]], yv)
        np.testing.assert_array_equal(ns[s, 0], sk)
        np.testing.assert_array_equal(ns[s, 1], sv)
    for s in (1, 3):          # untouched slots
        np.testing.assert_array_equal(ns[s], state[s])
