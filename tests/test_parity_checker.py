"""The parity checker the GPU tests use (``tests/parity.py``) must be able to
fail on the full-size workloads.  Here it is fed oracle results with a
plausible kernel mistake planted, at the 1M-key decode shape where outputs
are far below unit scale (|o| ~ 1e-2, lse ~ 15): one of 16 key splits lost
in the log-sum-exp merge (news article "vLLM, TML Inkling Day-0 support",
FA4 with sheared bias: the KV range is split per configuration and the
parts are merged).  It must reject those, and accept a result that differs
from the oracle only by the roundings a bf16 cache and bf16 output make."""


import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_attention, check_lse, check_out, check_out_scaled, check_p8

L = 1 << 20          # keys: the 1M-context full-attention decode
G = 8                # q-heads of one kv-head group
SPLITS = 16


@pytest.fixture(scope="module")
def decode_1m():
    """One sequence of the 1M decode shape, one kv-head group: the query at
    position L-1, full causal, R = L.  Returns inputs and the oracle's
    result as the merge of all 16 splits and with split 5 dropped."""
    rng = np.random.Generator(np.random.PCG64(5))
    q = synth.round_bf16(rng.standard_normal((1, G, 128), dtype=np.float32))
    bias = synth.round_bf16(rng.standard_normal((G, L), dtype=np.float32))
    K = synth.round_bf16(rng.standard_normal((L, 1, 128), dtype=np.float32)).astype(np.float64)
    V = synth.round_bf16(rng.standard_normal((L, 1, 128), dtype=np.float32)).astype(np.float64)
    pos = [L - 1]
    bounds = np.linspace(0, L, SPLITS + 1).astype(np.int64)
    parts = [oracle.relattn_rows(q, pos, K, V, bias, 0, G, key_lo=int(a), key_hi=int(b))
             for a, b in zip(bounds[:-1], bounds[1:])]
    full = oracle.lse_merge(parts)
    dropped = oracle.lse_merge(parts[:5] + parts[6:])
    return dict(q=q, bias=bias, K=K, V=V, full=full, dropped=dropped)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_checker_rejects_a_lost_split_at_1m(decode_1m, dtype):
    (o, l), (od, ld) = decode_1m["full"], decode_1m["dropped"]
    assert np.abs(o).max() < 2e-2        # far below unit scale: the elementwise bound alone is blind
    with pytest.raises(AssertionError):
        check_attention(od, o, ld, l, dtype, "dropped split", scale_aware=True)
    # each half of the check catches it on its own
    with pytest.raises(AssertionError):
        check_lse(ld, l, dtype)
    if dtype == "bf16":
        with pytest.raises(AssertionError):
            check_out_scaled(od, o)
    else:
        with pytest.raises(AssertionError):
            check_out(od, o, "fp32")


def test_checker_rejects_a_misweighted_split_at_1m(decode_1m):
    # a merge that averages the split outputs instead of weighting each by
    # exp(lse_s - lse): with splits of 1/16 and 15/16 of the keys the short
    # one gets weight 1/2 instead of about 1/16
    (o, l) = decode_1m["full"]
    q, K, V, bias = decode_1m["q"], decode_1m["K"], decode_1m["V"], decode_1m["bias"]
    cut = L // SPLITS
    a = oracle.relattn_rows(q, [L - 1], K, V, bias, 0, G, key_lo=0, key_hi=cut)
    b = oracle.relattn_rows(q, [L - 1], K, V, bias, 0, G, key_lo=cut, key_hi=L)
    wrong_o = 0.5 * (a[0] + b[0])                     # equal weights instead of lse weights
    with pytest.raises(AssertionError):
        check_attention(wrong_o, o, l, l, "bf16", "misweighted merge", scale_aware=True)


def test_checker_accepts_bf16_roundings_at_1m(decode_1m):
    # the oracle on the keys/values as a bf16 cache stores them (they are
    # bf16 values here already) with the output rounded to bf16 and lse
    # perturbed by the size of a logit rounding: a correct bf16 result
    (o, l) = decode_1m["full"]
    got_o = synth.round_bf16(o.astype(np.float32)).astype(np.float64)
    check_attention(got_o, o, l + 1e-3, l, "bf16", "rounded", scale_aware=True)


def test_checker_accepts_stored_kv_roundings_on_prefill_rows():
    # prefill rows of the 8K sliding-window shape: the oracle on fp64 K/V
    # against the oracle on the bf16-rounded K/V with its output rounded to
    # bf16 (the cache's and the output's roundings) passes every bound
    rng = np.random.Generator(np.random.PCG64(6))
    T, W = 4096, 2048
    q = synth.round_bf16(rng.standard_normal((T, G, 128), dtype=np.float32))
    bias = synth.round_bf16(rng.standard_normal((G, W), dtype=np.float32))
    K = rng.standard_normal((T, 1, 128))
    V = rng.standard_normal((T, 1, 128))
    rows = np.array([0, 1, 63, 64, 2047, 2048, 2049, 3000, T - 1])
    o, l = oracle.relattn_prefill(q, K, V, bias, W, G, rows=rows)
    Kb = synth.round_bf16(K.astype(np.float32)).astype(np.float64)
    Vb = synth.round_bf16(V.astype(np.float32)).astype(np.float64)
    ob, lb = oracle.relattn_prefill(q, Kb, Vb, bias, W, G, rows=rows)
    ob = synth.round_bf16(ob.astype(np.float32)).astype(np.float64)
    check_attention(ob, o, lb, l, "bf16", "stored kv", scale_aware=True)
    # and a 1/16 drop of the window's keys in one row is caught
    i = T - 1
    lo = i - W + 1
    cut = lo + W // 16
    part = oracle.relattn_rows(q[i:i + 1], [i], K, V, bias, W, G, key_lo=cut, key_hi=T)
    bad_o, bad_l = o.copy(), l.copy()
    bad_o[-1], bad_l[-1] = part[0][0], part[1][0]
    with pytest.raises(AssertionError):
        check_attention(bad_o, o, bad_l, l, "bf16", "dropped keys", scale_aware=True)
    assert np.isfinite(bad_l[-1]).all()


def _p8_case():
    rng = np.random.default_rng(11)
    L, T = 900, 48
    q = rng.standard_normal((T, 4, 128))
    K = rng.standard_normal((L, 1, 128))
    V = rng.standard_normal((L, 1, 128))
    bias = rng.standard_normal((4, 400)) * 0.5
    exp = oracle.relattn_prefill_p8_bounds(q, K, V, bias, 0, 4)
    return q, K, V, bias, exp


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def test_p8_checker_accepts_rounded_probabilities():
    # the exact result with the probabilities rounded to E4M3 at a random
    # running-maximum scale (oracle encoder) and the output rounded to bf16
    q, K, V, bias, exp = _p8_case()
    L, T = K.shape[0], q.shape[0]
    rng = np.random.default_rng(12)
    got_o = np.zeros_like(exp[0])
    got_l = np.zeros_like(exp[1])
    for r in range(T):
        i = L - T + r
        for h in range(4):
            s = K[:i + 1, 0] @ q[r, h] / np.sqrt(128) + bias[h, np.minimum(i - np.arange(i + 1), 399)]
            lam = 2.0 ** rng.uniform(0.0, 8.0)
            pr = oracle.fp8.e4m3_value(oracle.fp8.e4m3_code(lam * np.exp(s - s.max())))
            got_o[r, h] = (pr @ V[:i + 1, 0]) / pr.sum()
            got_l[r, h] = s.max() + np.log(pr.sum() / lam)
    check_p8(_bf16(got_o), got_l, exp)


def test_p8_checker_rejects_a_dropped_key_tile():
    # the oracle's own result without one 64-key tile in the middle of the keys
    q, K, V, bias, exp = _p8_case()
    L, T = K.shape[0], q.shape[0]
    parts = [oracle.relattn_rows(q, np.arange(L - T, L), K, V, bias, 0, 4, key_lo=0, key_hi=384),
             oracle.relattn_rows(q, np.arange(L - T, L), K, V, bias, 0, 4, key_lo=448)]
    o, l = oracle.lse_merge(parts)
    with pytest.raises(AssertionError):
        check_p8(_bf16(o), l, exp)
