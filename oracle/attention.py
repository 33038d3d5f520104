"""Relative-position grouped-query attention -- fp64 oracle.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:

* news article "vLLM, TML Inkling Day-0 support", *Model Architecture /
  Attention*: every attention layer is grouped-query attention with head size
  128; most layers attend over a sliding window, the rest over the full causal
  prefix; instead of RoPE a learned relative-position term is added to the
  logits before the softmax.  Recipe "thinkingmachines/Inkling", *Guide /
  Overview*, says the same.
* same article, *FA4 with sheared bias*: the attention kernel splits the KV
  range into a per-configuration number of parts.  Splitting is only correct
  because softmax attention over a union of key sets is the log-sum-exp
  weighted combination of the attention over each part (:func:`lse_merge`).

Readings where the pages are silent (each listed in the design notes):

* logit[h, i, j] = (q_i . k_j) / sqrt(d) + bias[h][min(i - j, R - 1)], with one
  bias row per *query* head; the scale applies to q.k only; natural-exp
  softmax;
* query i sees key j iff j <= i and, for a window W > 0, i - j <= W - 1 (W keys
  including itself); W = 0 means full causal;
* query head h reads KV head h // (Hq / Hkv);
* positions start at 0 in each sequence; a chunk of q_len queries occupies the
  last q_len positions of a sequence of seq_len keys.

Output ``lse`` is the natural log of the softmax denominator including the
running max, i.e. log(sum_j exp(logit_j)).
"""

import math

import numpy as np


def visible_key_range(i, window):
    """Inclusive range [lo, hi] of key positions visible to query position i."""
    lo = 0 if window == 0 else max(0, i - window + 1)
    return lo, i


def relattn_rows(q_rows, positions, K, V, bias, window, num_q_heads_per_kv,
                 key_lo=0, key_hi=None):
    """Attention for a set of query rows of one sequence.

    q_rows    : [n, Hq, d] queries.
    positions : [n] logical position of each query row.
    K, V      : [L, Hkv, d] keys / values of positions 0..L-1.
    bias      : [Hq, R] relative-position table.
    window    : W (0 = full causal).
    num_q_heads_per_kv : Hq // Hkv.
    key_lo, key_hi : restrict the keys additionally to [key_lo, key_hi)
                (used to form the partial results that :func:`lse_merge`
                combines); defaults to all keys.

    Returns (out [n, Hq, d], lse [n, Hq]) in float64.  A row with no visible
    key in the restricted range has out = 0 and lse = -inf.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    n, Hq, d = q_rows.shape
    L = K.shape[0]
    R = bias.shape[1]
    if key_hi is None:
        key_hi = L
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, Hq, d))
    lse = np.full((n, Hq), -np.inf)
    for r in range(n):
        i = int(positions[r])
        lo, hi = visible_key_range(i, window)
        lo, hi = max(lo, key_lo), min(hi, key_hi - 1)
        if hi < lo:
            continue
        j = np.arange(lo, hi + 1)
        dist = np.minimum(i - j, R - 1)
        for h in range(Hq):
            g = h // num_q_heads_per_kv
            s = (K[lo:hi + 1, g, :] @ q_rows[r, h]) * scale + bias[h, dist]
            m = s.max()
            e = np.exp(s - m)
            den = e.sum()
            out[r, h] = (e @ V[lo:hi + 1, g, :]) / den
            lse[r, h] = m + math.log(den)
    return out, lse


def _block_logits(Q, K, bias_h, positions, window, key_lo, key_hi):
    """Logits [rows, keys] of one query head for keys key_lo .. key_hi-1, -inf
    where a key is not visible (the definition of :func:`relattn_rows`)."""
    i = positions[:, None]
    j = np.arange(key_lo, key_hi)[None, :]
    R = bias_h.shape[0]
    d = Q.shape[1]
    dist = i - j
    visible = dist >= 0
    if window > 0:
        visible &= dist <= window - 1
    logits = (Q @ K[key_lo:key_hi].T) / math.sqrt(d)
    logits = logits + bias_h[np.clip(dist, 0, R - 1)]
    return np.where(visible, logits, -np.inf)


def _relattn_block(Q, K, V, bias_h, positions, window, key_lo, key_hi):
    """Same definition as :func:`relattn_rows` for one query head and a block
    of rows, written as matrix products (rows are still independent)."""
    logits = _block_logits(Q, K, bias_h, positions, window, key_lo, key_hi)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=1, keepdims=True)
    return (e @ V[key_lo:key_hi]) / den, (m + np.log(den))[:, 0]


def relattn_prefill(q, K, V, bias, window, num_q_heads_per_kv, q_start=None,
                    rows=None, row_block=256):
    """Prefill attention for one sequence chunk.

    q : [T, Hq, d] queries of the chunk; K, V : [L, Hkv, d] all keys of the
    sequence (L >= T).  The chunk sits at positions q_start .. q_start+T-1,
    by default the last T positions (q_start = L - T).

    rows : optional subset of chunk rows to evaluate (others are not
    computed); returns (out [len(rows), Hq, d], lse [len(rows), Hq]).
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    L = K.shape[0]
    if q_start is None:
        q_start = L - T
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, d))
    lse = np.zeros((len(rows), Hq))
    for c0 in range(0, len(rows), row_block):
        sel = rows[c0:c0 + row_block]
        pos = q_start + sel
        lo = 0 if window == 0 else max(0, int(pos.min()) - window + 1)
        hi = int(pos.max()) + 1
        for h in range(Hq):
            g = h // num_q_heads_per_kv
            Qb = q[sel, h, :].astype(np.float64)
            o, l = _relattn_block(Qb, K[:, g, :], V[:, g, :], bias[h], pos,
                                  window, lo, hi)
            out[c0:c0 + len(sel), h] = o
            lse[c0:c0 + len(sel), h] = l
    return out, lse


def relattn_prefill_p8_bounds(q, K, V, bias, window, num_q_heads_per_kv, q_start=None,
                              rows=None, row_block=256):
    """:func:`relattn_prefill` plus the error that rounding the softmax
    probabilities to E4M3 (ties to even, row sums over the rounded values)
    can cause, for FP8 matrix products.

    With p_j = exp(logit_j - max) and a kernel running maximum anywhere in
    [max - 8 ln 2, max] (so its probabilities are lambda * p_j, 1 <= lambda
    <= 256), the rounding moves lambda * p_j by at most half an E4M3 step,
    which relative to the row sum lambda * sum p is at most
    h_j = max(p_j / 8, 2^-9) / 2 / sum p (the step is at most a value's 1/8
    among normals, and 2^-9 among subnormals).  The output O = sum w_j v_j
    then moves by sum_j e_j (v_j - O) / sum p^ with |e_j| <= h_j sum p, so

      bound_o = sum_j h_j |v_j - O| / (1 - sum_j h_j)        (per dimension)
      sigma_o = sqrt(sum_j h_j^2 / 3 (v_j - O)^2)            (errors uniform
                                                              in +-h_j)
      bound_l = -log(1 - sum_j h_j),  sigma_l = sqrt(sum_j h_j^2 / 3)

    for the log-sum-exp.  Returns (out, lse, bound_o, sigma_o, bound_l,
    sigma_l), shapes as :func:`relattn_prefill` ([rows, Hq, d] and [rows, Hq]).
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    L = K.shape[0]
    if q_start is None:
        q_start = L - T
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    out, bo, so = (np.zeros((n, Hq, d)) for _ in range(3))
    lse, bl, sl = (np.zeros((n, Hq)) for _ in range(3))
    for c0 in range(0, n, row_block):
        sel = rows[c0:c0 + row_block]
        pos = q_start + sel
        lo = 0 if window == 0 else max(0, int(pos.min()) - window + 1)
        hi = int(pos.max()) + 1
        for h in range(Hq):
            g = h // num_q_heads_per_kv
            logits = _block_logits(q[sel, h, :].astype(np.float64), K[:, g, :], bias[h], pos,
                                   window, lo, hi)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            den = p.sum(axis=1, keepdims=True)
            Vb = V[lo:hi, g, :]
            o = (p @ Vb) / den
            hrel = np.where(p > 0, np.maximum(p / 8.0, 2.0 ** -9) / 2.0, 0.0) / den
            hsum = hrel.sum(axis=1)
            # sum_j h_j |v_j - O|, over blocks of rows and keys (memory)
            babs = np.zeros_like(o)
            for r0 in range(0, len(sel), 32):
                for k0 in range(0, Vb.shape[0], 512):
                    dev = np.abs(Vb[None, k0:k0 + 512, :] - o[r0:r0 + 32, None, :])
                    babs[r0:r0 + 32] += np.einsum("rk,rkd->rd", hrel[r0:r0 + 32, k0:k0 + 512], dev)
            # sum_j a_j (v_j - O)^2 = sum a v^2 - 2 O sum a v + O^2 sum a
            a = hrel ** 2 / 3.0
            var = a @ (Vb * Vb) - 2.0 * o * (a @ Vb) + o * o * a.sum(axis=1, keepdims=True)
            sl_ = slice(c0, c0 + len(sel))
            out[sl_, h] = o
            lse[sl_, h] = (m + np.log(den))[:, 0]
            bo[sl_, h] = babs / (1.0 - hsum)[:, None]
            so[sl_, h] = np.sqrt(np.maximum(var, 0.0))
            bl[sl_, h] = -np.log1p(-hsum)
            sl[sl_, h] = np.sqrt((hrel ** 2 / 3.0).sum(axis=1))
    return out, lse, bo, so, bl, sl


def relattn_decode(q, K, V, bias, window, num_q_heads_per_kv):
    """One decode step of one sequence: the query at position L-1 (the token
    just appended, whose key and value are K[L-1], V[L-1]).

    q : [Hq, d]; K, V : [L, Hkv, d].  Returns (out [Hq, d], lse [Hq]).
    """
    L = np.asarray(K).shape[0]
    out, lse = relattn_rows(np.asarray(q)[None], [L - 1], K, V, bias, window,
                            num_q_heads_per_kv)
    return out[0], lse[0]


def lse_merge(parts):
    """Combine attention results over disjoint key sets.

    parts : iterable of (out_s [..., d], lse_s [...]); a part whose lse is
    -inf saw no key and contributes nothing.

        lse = log sum_s exp(lse_s),   out = sum_s exp(lse_s - lse) * out_s
    """
    parts = list(parts)
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    m = lses.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - safe_m)                      # exp(-inf) = 0
    den = w.sum(axis=0)
    lse = safe_m + np.log(den)
    out = (w[..., None] * outs).sum(axis=0) / den[..., None]
    return out, lse
