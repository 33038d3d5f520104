"""Pins of the oracle pieces behind FP8 matrix products (CPU only).

* ``quantize_query_tiles``: codes equal torch's ``float8_e4m3fn`` cast of
  fp32(q) * fp32(448 / amax) (a library implementation of the rounding); the
  largest element of a tile reads back as itself; tiles are independent and
  start at row 0 of each sequence's chunk; an all-zero tile reads back as 0.
* ``e4m3_spacing``: the gaps between consecutive E4M3 values, from the code
  table (itself pinned to torch in ``test_oracle_fp8``).
* ``relattn_prefill_p8_bounds``: its output and lse are ``relattn_prefill``'s;
  closed forms for one visible key and for equal logits; and a Monte Carlo
  run that rounds the probabilities to E4M3 (the oracle's encoder) at random
  running-maximum scales stays inside ``bound`` and has errors of the size
  ``sigma`` predicts.
"""

import math

import numpy as np
import torch

import oracle
import oracle.fp8 as fp8


def _torch_code(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _q(rng, n, H=3):
    return (rng.standard_normal((n, H, 128)) * rng.uniform(0.1, 5.0, (1, H, 1))).astype(np.float32)


def test_query_codes_match_torch_cast():
    rng = np.random.default_rng(0)
    q = _q(rng, 700)
    cu = [0, 300, 301, 700]
    back, codes = fp8.quantize_query_tiles(q, cu)
    for b in range(3):
        for r0 in range(cu[b], cu[b + 1], 256):
            r1 = min(r0 + 256, cu[b + 1])
            for h in range(q.shape[1]):
                x = q[r0:r1, h]
                amax = np.float32(np.abs(x).max())
                inv = np.float32(448.0) / amax
                want = _torch_code(x * inv)
                assert np.array_equal(codes[r0:r1, h], want)
                s = float(np.float32(amax / np.float32(448.0)))
                vals = torch.from_numpy(want).view(torch.float8_e4m3fn).to(torch.float64).numpy()
                assert np.array_equal(back[r0:r1, h], vals * s)


def test_tile_max_reads_back_as_itself_and_error_is_within_half_a_step():
    rng = np.random.default_rng(1)
    q = _q(rng, 512, H=2)
    back, codes = fp8.quantize_query_tiles(q, [0, 512])
    for r0 in (0, 256):
        for h in range(2):
            x = q[r0:r0 + 256, h].astype(np.float64)
            i = np.unravel_index(np.abs(x).argmax(), x.shape)
            assert codes[r0:r0 + 256, h][i] & 0x7F == 0x7E          # 448
            assert abs(back[r0:r0 + 256, h][i] - x[i]) <= 1e-6 * abs(x[i])
            s = np.abs(x).max() / 448.0
            half = fp8.e4m3_spacing(x / s) / 2 * s
            assert np.all(np.abs(back[r0:r0 + 256, h] - x) <= half * (1 + 1e-6) + 1e-12)


def test_tiles_are_independent_and_start_at_each_chunk():
    rng = np.random.default_rng(2)
    q = _q(rng, 600, H=2)
    cu = [0, 270, 600]                 # tiles: [0,256) [256,270) [270,526) [526,600)
    base, _ = fp8.quantize_query_tiles(q, cu)
    q2 = q.copy()
    q2[260, 1] *= 100.0                # inside the second tile, head 1
    got, _ = fp8.quantize_query_tiles(q2, cu)
    changed = np.any(got != base, axis=2)
    assert changed[256:270, 1].all()
    changed[256:270, 1] = False
    assert not changed.any()
    z = q.copy()
    z[270:526, 0] = 0.0
    zb, zc = fp8.quantize_query_tiles(z, cu)
    assert not zb[270:526, 0].any() and not zc[270:526, 0].any()


def test_spacing_is_the_gap_between_codes():
    mags = fp8.e4m3_value(np.arange(0x7F))          # ascending finite magnitudes
    gaps = np.diff(mags)
    assert np.array_equal(fp8.e4m3_spacing(mags[:-1]), gaps)
    assert np.array_equal(fp8.e4m3_spacing(-mags[:-1]), gaps)


def _case(rng, L=300, T=40, Hq=4, Hkv=2, R=50):
    q = rng.standard_normal((T, Hq, 128))
    K = rng.standard_normal((L, Hkv, 128))
    V = rng.standard_normal((L, Hkv, 128))
    bias = rng.standard_normal((Hq, R))
    return q, K, V, bias


def test_bounds_carry_the_exact_attention():
    rng = np.random.default_rng(3)
    q, K, V, bias = _case(rng)
    for W in (0, 64):
        o, l, *_ = oracle.relattn_prefill_p8_bounds(q, K, V, bias, W, 2)
        o2, l2 = oracle.relattn_prefill(q, K, V, bias, W, 2)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_bounds_closed_forms():
    rng = np.random.default_rng(4)
    q, K, V, bias = _case(rng, L=200, T=200)
    # row 0 sees one key: nothing to round against
    o, l, bo, so, bl, sl = oracle.relattn_prefill_p8_bounds(q, K, V, bias, 0, 2)
    assert not bo[0].any() and np.all(so[0] < 1e-7)
    assert abs(bl[0, 0] - (-math.log1p(-1 / 16))) < 1e-12          # p = 1 -> h = 1/16
    # equal logits (q = 0, constant bias): every p_j = 1 over the N visible keys
    q0 = np.zeros_like(q)
    b0 = np.full_like(bias, 0.7)
    o, l, bo, so, bl, sl = oracle.relattn_prefill_p8_bounds(q0, K, V, b0, 0, 2)
    for r in (5, 77, 199):
        N = r + 1
        v = V[:N, 1, :]
        mean = v.mean(axis=0)
        assert np.allclose(bo[r, 3], np.abs(v - mean).sum(axis=0) / (16 * N) / (1 - 1 / 16))
        assert np.allclose(so[r, 3], np.sqrt(((v - mean) ** 2).sum(axis=0) / 3) / (16 * N))
        assert np.isclose(bl[r, 3], -math.log1p(-1 / 16))
        assert np.isclose(sl[r, 3], math.sqrt(N / 3) / (16 * N))


def test_bounds_cover_rounded_probabilities():
    # Round lambda * p_j to E4M3 (oracle encoder) for running maxima anywhere
    # in [max - 8 ln 2, max], take the weighted mean over the rounded values,
    # and check it against the bound and the predicted spread.
    rng = np.random.default_rng(5)
    L, T = 700, 60
    q, K, V, bias = _case(rng, L=L, T=T, Hq=2, Hkv=1, R=300)
    q *= 2.0                            # peakier rows as well as diffuse ones
    o, l, bo, so, bl, sl = oracle.relattn_prefill_p8_bounds(q, K, V, bias, 0, 2)
    z_o, z_l = [], []
    for r in range(T):
        i = L - T + r
        for h in range(2):
            s = K[:i + 1, 0] @ q[r, h] / math.sqrt(128) + bias[h, np.minimum(i - np.arange(i + 1), 299)]
            p = np.exp(s - s.max())
            lam = 2.0 ** rng.uniform(0.0, 8.0)
            pr = fp8.e4m3_value(fp8.e4m3_code(lam * p))
            got = (pr @ V[:i + 1, 0]) / pr.sum()
            gl = s.max() + math.log(pr.sum() / lam)
            err = got - o[r, h]
            assert np.all(np.abs(err) <= bo[r, h] * (1 + 1e-9) + 1e-12)
            assert abs(gl - l[r, h]) <= bl[r, h] * (1 + 1e-9) + 1e-12
            z_o.append(err / np.maximum(so[r, h], 1e-300))
            z_l.append((gl - l[r, h]) / max(sl[r, h], 1e-300))
    rms_o = math.sqrt(np.mean(np.concatenate(z_o) ** 2))
    rms_l = math.sqrt(np.mean(np.array(z_l) ** 2))
    assert rms_o < 1.5 and rms_l < 1.5, (rms_o, rms_l)
