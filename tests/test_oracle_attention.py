"""Pins of the attention oracle against things other than itself.

The pages give no formula or worked example for the relative term, so the
oracle is pinned by:

* library routines: torch float64 ``scaled_dot_product_attention`` on the CPU
  with a boolean causal/window mask (zero bias) and with an additive float
  mask (any bias);
* closed forms: with q = 0 the logits are the bias alone, and a bias that is
  linear in the distance gives a truncated geometric distribution whose mean
  is known in closed form -- this fixes the sign and offset of the distance
  index and the window width; lse = log(#visible keys) for zero logits; two
  visible keys give a logistic weight;
* metamorphic invariants named by the method: window >= T is full causal,
  GQA equals MHA with replicated KV heads, a per-head constant bias changes
  nothing, constant V passes through, clipping at R-1 equals a table extended
  with its last entry, block-table permutations change nothing, decode with
  the sconv cache equals prefill of the same tokens, and the log-sum-exp
  merge of any key partition equals the unsplit result;
* a pure-Python brute force on tiny inputs.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

RNG = np.random.default_rng


def _qkv(T, Hq, Hkv, d, seed=0, L=None):
    rng = RNG(seed)
    L = T if L is None else L
    return (rng.standard_normal((T, Hq, d)), rng.standard_normal((L, Hkv, d)),
            rng.standard_normal((L, Hkv, d)))


def _sdpa(q, K, V, mask):
    """torch float64 SDPA; q [T,H,d], K/V [L,H,d], mask [H,T,L] (bool or float)."""
    qt = torch.from_numpy(q.transpose(1, 0, 2).copy())[None]
    kt = torch.from_numpy(K.transpose(1, 0, 2).copy())[None]
    vt = torch.from_numpy(V.transpose(1, 0, 2).copy())[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None])
    return o[0].numpy().transpose(1, 0, 2)


def _bool_mask(T, L, W):
    i = np.arange(L - T, L)[:, None]
    j = np.arange(L)[None, :]
    m = j <= i
    if W > 0:
        m &= (i - j) <= W - 1
    return m


@pytest.mark.parametrize("W", [0, 1, 5, 40])
def test_zero_bias_equals_library_softmax_attention(W):
    T, H, d = 40, 3, 128
    q, K, V = _qkv(T, H, H, d, seed=1)
    out, _ = oracle.relattn_prefill(q, K, V, np.zeros((H, 8)), W, 1)
    mask = np.broadcast_to(_bool_mask(T, T, W), (H, T, T)).copy()
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask), atol=1e-12)


@pytest.mark.parametrize("W,R", [(0, 64), (7, 64), (0, 5), (12, 3)])
def test_any_bias_equals_library_attention_with_additive_mask(W, R):
    T, H, d = 24, 2, 128
    q, K, V = _qkv(T, H, H, d, seed=2)
    bias = RNG(3).standard_normal((H, R))
    out, _ = oracle.relattn_prefill(q, K, V, bias, W, 1)
    # Additive mask built entry by entry from the table (library does the rest).
    allowed = _bool_mask(T, T, W)
    mask = np.full((H, T, T), -np.inf)
    for h in range(H):
        for i in range(T):
            for j in range(T):
                if allowed[i, j]:
                    mask[h, i, j] = bias[h, min(i - j, R - 1)]
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask), atol=1e-12)


@pytest.mark.parametrize("W", [0, 6])
def test_linear_bias_geometric_closed_form(W):
    # q = 0 => logits = bias only. With bias[r] = -alpha * r, the weight of key
    # j at distance r = i - j is rho^r / sum rho^r (rho = e^-alpha), truncated
    # at n = #visible keys. With v_j = j the output is i - E[r] where
    #   E[r] = rho/(1-rho) - n rho^n / (1 - rho^n).
    T, d, alpha = 20, 128, 0.7
    rho = math.exp(-alpha)
    R = 64
    bias = (-alpha * np.arange(R))[None, :]
    q = np.zeros((T, 1, d))
    K = RNG(4).standard_normal((T, 1, d))
    V = np.zeros((T, 1, d))
    V[:, 0, 0] = np.arange(T)
    V[:, 0, 1] = 1.0
    out, lse = oracle.relattn_prefill(q, K, V, bias, W, 1)
    for i in range(T):
        n = i + 1 if W == 0 else min(i + 1, W)
        er = rho / (1 - rho) - n * rho ** n / (1 - rho ** n)
        assert out[i, 0, 0] == pytest.approx(i - er, abs=1e-12)
        assert out[i, 0, 1] == pytest.approx(1.0, abs=1e-14)
        assert lse[i, 0] == pytest.approx(math.log((1 - rho ** n) / (1 - rho)), abs=1e-12)


def test_zero_logits_lse_is_log_count():
    T, d, W = 30, 128, 9
    q = np.zeros((T, 2, d))
    K, V = RNG(5).standard_normal((2, T, 1, d))
    _, lse = oracle.relattn_prefill(q, K, V, np.zeros((2, 4)), W, 2)
    n = np.minimum(np.arange(T) + 1, W)
    np.testing.assert_allclose(lse, np.log(n)[:, None].repeat(2, 1), atol=1e-13)


def test_two_keys_logistic_weight():
    # Row 1 of a causal sequence sees keys 0 and 1 only.
    d = 128
    q = np.zeros((2, 1, d)); q[1, 0, 0] = math.sqrt(d)       # q.k/sqrt(d) = k[0]
    K = np.zeros((2, 1, d)); K[0, 0, 0] = 0.3; K[1, 0, 0] = -0.9
    V = np.zeros((2, 1, d)); V[0, 0, 5] = 1.0; V[1, 0, 6] = 1.0
    bias = np.array([[0.25, -0.5, 7.0]])                      # dist 0, 1, 2
    out, _ = oracle.relattn_prefill(q, K, V, bias, 0, 1)
    a = 0.3 + (-0.5)        # key 0: distance 1
    b = -0.9 + 0.25         # key 1: distance 0
    p0 = 1.0 / (1.0 + math.exp(b - a))
    assert out[1, 0, 5] == pytest.approx(p0, abs=1e-15)
    assert out[1, 0, 6] == pytest.approx(1 - p0, abs=1e-15)


def test_window_ge_T_is_full_causal():
    T, H, d = 33, 2, 128
    q, K, V = _qkv(T, H, 1, d, seed=6)
    bias = RNG(7).standard_normal((H, 50))
    full, lf = oracle.relattn_prefill(q, K, V, bias, 0, 2)
    for W in (T, T + 1, 1000):
        o, l = oracle.relattn_prefill(q, K, V, bias, W, 2)
        np.testing.assert_array_equal(o, full)
        np.testing.assert_array_equal(l, lf)


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 2), (8, 4)])
def test_gqa_equals_mha_with_replicated_kv(Hq, Hkv):
    T, d = 21, 128
    q, K, V = _qkv(T, Hq, Hkv, d, seed=8)
    bias = RNG(9).standard_normal((Hq, 16))
    g = Hq // Hkv
    o_gqa, l_gqa = oracle.relattn_prefill(q, K, V, bias, 11, g)
    Kr = np.repeat(K, g, axis=1)
    Vr = np.repeat(V, g, axis=1)
    o_mha, l_mha = oracle.relattn_prefill(q, Kr, Vr, bias, 11, 1)
    np.testing.assert_allclose(o_gqa, o_mha, atol=1e-14)
    np.testing.assert_allclose(l_gqa, l_mha, atol=1e-14)


def test_constant_bias_per_head_is_shift_invariant():
    T, H, d = 17, 3, 128
    q, K, V = _qkv(T, H, H, d, seed=10)
    o0, l0 = oracle.relattn_prefill(q, K, V, np.zeros((H, 9)), 5, 1)
    c = np.array([1.5, -2.0, 30.0])
    o1, l1 = oracle.relattn_prefill(q, K, V, np.tile(c[:, None], (1, 9)), 5, 1)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1 - l0, np.tile(c, (T, 1)), atol=1e-12)


def test_constant_v_and_first_row():
    T, H, d = 12, 2, 128
    q, K, V = _qkv(T, H, 1, d, seed=11)
    bias = RNG(12).standard_normal((H, 12))
    vc = RNG(13).standard_normal(d)
    Vc = np.tile(vc, (T, 1, 1))
    o, _ = oracle.relattn_prefill(q, K, Vc, bias, 0, 2)
    np.testing.assert_allclose(o, np.broadcast_to(vc, o.shape), atol=1e-14)
    o, l = oracle.relattn_prefill(q, K, V, bias, 0, 2)
    np.testing.assert_allclose(o[0], np.tile(V[0], (2, 1)), atol=1e-15)
    # row 0 sees one key at distance 0: lse = q0.k0/sqrt(d) + bias[h][0]
    for h in range(H):
        assert l[0, h] == pytest.approx(q[0, h] @ K[0, 0] / math.sqrt(d) + bias[h, 0])


def _brute(q, K, V, bias, W, g):
    T, Hq, d = len(q), len(q[0]), len(q[0][0])
    R = len(bias[0])
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(T)]
    for i in range(T):
        for h in range(Hq):
            kv = h // g
            logits = []
            for j in range(T):
                if j > i or (W > 0 and i - j > W - 1):
                    continue
                s = 0.0
                for c in range(d):
                    s += q[i][h][c] * K[j][kv][c]
                logits.append((j, s / math.sqrt(d) + bias[h][min(i - j, R - 1)]))
            m = max(s for _, s in logits)
            den = sum(math.exp(s - m) for _, s in logits)
            for c in range(d):
                out[i][h][c] = sum(math.exp(s - m) * V[j][kv][c] for j, s in logits) / den
    return np.array(out)


@pytest.mark.parametrize("T,W,R", [(16, 0, 16), (16, 4, 8), (9, 3, 2), (1, 0, 1)])
def test_pure_python_brute_force(T, W, R):
    Hq, Hkv, d = 4, 2, 128
    q, K, V = _qkv(T, Hq, Hkv, d, seed=14)
    bias = RNG(15).standard_normal((Hq, R))
    o, _ = oracle.relattn_prefill(q, K, V, bias, W, Hq // Hkv)
    ob = _brute(q.tolist(), K.tolist(), V.tolist(), bias.tolist(), W, Hq // Hkv)
    np.testing.assert_allclose(o, ob, atol=1e-12)


def test_clip_equals_extended_table():
    T, H, d, W = 48, 2, 128, 40
    q, K, V = _qkv(T, H, H, d, seed=16)
    R = 16
    bias = RNG(17).standard_normal((H, R))
    ext = np.concatenate([bias, np.repeat(bias[:, -1:], 100, axis=1)], axis=1)
    o1, l1 = oracle.relattn_prefill(q, K, V, bias, W, 1)
    o2, l2 = oracle.relattn_prefill(q, K, V, ext, W, 1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_blocked_prefill_equals_per_row_definition():
    T, Hq, Hkv, d = 70, 4, 2, 128
    q, K, V = _qkv(T, Hq, Hkv, d, seed=18, L=90)
    bias = RNG(19).standard_normal((Hq, 30))
    o1, l1 = oracle.relattn_prefill(q, K, V, bias, 25, 2, row_block=16)
    o2, l2 = oracle.relattn_rows(q, np.arange(20, 90), K, V, bias, 25, 2)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_causality_future_keys_do_not_matter():
    T, H, d = 25, 2, 128
    q, K, V = _qkv(T, H, 1, d, seed=20)
    bias = RNG(21).standard_normal((H, 25))
    o1, _ = oracle.relattn_prefill(q, K, V, bias, 0, 2)
    K2, V2 = K.copy(), V.copy()
    K2[13:] += 5.0
    V2[13:] -= 3.0
    o2, _ = oracle.relattn_prefill(q, K2, V2, bias, 0, 2)
    np.testing.assert_array_equal(o1[:13], o2[:13])


@pytest.mark.parametrize("parts", [[0, 50], [0, 1, 50], [0, 7, 14, 21, 28, 35, 42, 50],
                                   [0, 3, 4, 49, 50], [0, 10, 11, 50]])
@pytest.mark.parametrize("W", [0, 9])
def test_lse_merge_of_any_partition_equals_unsplit(parts, W):
    L, Hq, d = 50, 4, 128
    q, K, V = _qkv(L, Hq, 2, d, seed=22)
    bias = RNG(23).standard_normal((Hq, 64))
    rows = np.arange(L)
    o, l = oracle.relattn_rows(q, rows, K, V, bias, W, 2)
    pieces = [oracle.relattn_rows(q, rows, K, V, bias, W, 2, key_lo=a, key_hi=b)
              for a, b in zip(parts[:-1], parts[1:])]
    om, lm = oracle.lse_merge(pieces)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)


def test_block_table_permutation_invariance():
    c1 = synth.make_case("fp32", [1], [300], 4, 1, 0, 400, seed=24, extra_blocks=3)
    store = oracle.PagedStore(c1.num_blocks, 1, 128)
    store.k[:] = c1.past_k
    store.v[:] = c1.past_v
    K, V = store.gather(c1.block_table[0], 301)
    o1, l1 = oracle.relattn_decode(c1.q[0], K, V, c1.bias, 0, 4)
    # move every block to a new physical place
    perm = RNG(25).permutation(c1.num_blocks)
    store2 = oracle.PagedStore(c1.num_blocks, 1, 128)
    for old in range(c1.num_blocks):
        new = perm[old]
        store2.k[new * 128:(new + 1) * 128] = store.k[old * 128:(old + 1) * 128]
        store2.v[new * 128:(new + 1) * 128] = store.v[old * 128:(old + 1) * 128]
    table2 = perm[c1.block_table[0]]
    K2, V2 = store2.gather(table2, 301)
    o2, l2 = oracle.relattn_decode(c1.q[0], K2, V2, c1.bias, 0, 4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("W", [0, 20])
def test_decode_with_sconv_cache_equals_prefill(W):
    # Prefill P tokens, then decode the remaining tokens one by one carrying
    # the sconv state and the paged cache; every decoded row must equal the
    # corresponding row of a single prefill over all tokens.
    T, P, Hq, Hkv, d = 40, 29, 4, 2, 128
    C = Hkv * d
    c = synth.make_case("fp32", [T], [0], Hq, Hkv, W, 32, seed=26, extra_blocks=2)
    w = c.conv_w
    # one-shot prefill
    ko, vo, st_full = oracle.sconv_batch(c.k_pre, c.v_pre, w, c.conv_state,
                                         c.state_slot, c.cu_seqlens)
    K = ko.reshape(T, Hkv, d)
    V = vo.reshape(T, Hkv, d)
    o_ref, l_ref = oracle.relattn_prefill(c.q, K, V, c.bias, W, Hq // Hkv)
    # incremental: prefill of P tokens, then T-P decode steps through the cache
    store = oracle.PagedStore(c.num_blocks, Hkv, d)
    table = c.block_table[0]
    state = c.conv_state.astype(np.float64)
    kp, vp, state = oracle.sconv_batch(c.k_pre[:P], c.v_pre[:P], w, state,
                                       [0], [0, P])
    store.write(oracle.slots_for(table, np.arange(P)), kp.reshape(P, Hkv, d),
                vp.reshape(P, Hkv, d))
    Kc, Vc = store.gather(table, P)
    o_p, _ = oracle.relattn_prefill(c.q[:P], Kc, Vc, c.bias, W, Hq // Hkv)
    np.testing.assert_allclose(o_p, o_ref[:P], atol=1e-12)
    for t in range(P, T):
        kt, vt, state = oracle.sconv_batch(c.k_pre[t:t + 1], c.v_pre[t:t + 1], w,
                                           state, [0], [0, 1])
        store.write([oracle.slot_of(table, t)], kt.reshape(1, Hkv, d),
                    vt.reshape(1, Hkv, d))
        Kc, Vc = store.gather(table, t + 1)
        o, l = oracle.relattn_decode(c.q[t], Kc, Vc, c.bias, W, Hq // Hkv)
        np.testing.assert_allclose(o, o_ref[t], atol=1e-12)
        np.testing.assert_allclose(l, l_ref[t], atol=1e-12)
    np.testing.assert_allclose(state, st_full, atol=0)
    assert C == 256
