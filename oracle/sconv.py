"""Short convolution (sconv) with its three-token state cache -- fp64 oracle.

Test infrastructure only (see ``oracle/__init__.py``).

Source: news article "vLLM, TML Inkling Day-0 support", *Model Architecture /
Sconv* (window-4 short convolution applied, among others, to the attention keys
and values, channel by channel) and *vLLM Integration & Optimization /
Managing the sconv cache* (the cache keeps the hidden states of the last W-1
tokens, W = 4).  Recipe "thinkingmachines/Inkling", *Guide / Overview*, repeats
both facts.

Readings where the pages are silent (each listed in the design notes):

* causal taps including the current token: tap 3 multiplies x[t], tap 0
  multiplies x[t-3] (a depthwise convolution with 3 zeros of left padding);
* no bias, activation, residual or normalisation: a pure linear map;
* the cached "hidden states" are the *pre-convolution* inputs of the last
  three tokens, zero for a fresh sequence; after a chunk of n tokens the new
  state is the last three rows of [old state; chunk], which also covers n < 3.
"""

import numpy as np

WIDTH = 4            # convolution window W
STATE_ROWS = WIDTH - 1


def sconv_sequence(x, w, state=None):
    """Convolve one sequence chunk.

    x     : [n, C] pre-convolution inputs of the chunk, oldest token first.
    w     : [C, 4] per-channel taps; w[c, 3] weights the current token.
    state : [3, C] pre-convolution inputs of the three tokens before the
            chunk (oldest first), or None for a fresh sequence (zeros).

    Returns (y [n, C], new_state [3, C]) in float64, where
        y[t, c] = sum_{k=0..3} w[c, k] * xp[t + k, c],  xp = [state; x],
    and new_state = the last three rows of xp.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n, C = x.shape
    assert w.shape == (C, WIDTH)
    if state is None:
        state = np.zeros((STATE_ROWS, C))
    state = np.asarray(state, dtype=np.float64)
    assert state.shape == (STATE_ROWS, C)
    xp = np.concatenate([state, x], axis=0)          # [n + 3, C]
    y = np.zeros((n, C))
    for k in range(WIDTH):
        y += w[:, k][None, :] * xp[k:k + n]
    new_state = xp[n:n + STATE_ROWS].copy()
    return y, new_state


def sconv_batch(k_in, v_in, conv_w, conv_state, state_slot, cu_seqlens):
    """Sconv over a ragged batch of sequence chunks, keys and values apart.

    k_in, v_in : [N_tok, C] pre-convolution keys / values (C = Hkv * d),
                 sequences packed back to back.
    conv_w     : [2, C, 4] taps, [0] for keys and [1] for values.
    conv_state : [num_slots, 2, 3, C] per-sequence cache of pre-convolution
                 inputs ([.,0] keys, [.,1] values).
    state_slot : [num_seqs] row of conv_state owned by each sequence.
    cu_seqlens : [num_seqs + 1] token offsets of the sequences.

    Returns (k_out, v_out, new_conv_state) in float64; rows of conv_state not
    named by state_slot are returned unchanged.
    """
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    conv_w = np.asarray(conv_w, dtype=np.float64)
    new_state = np.array(conv_state, dtype=np.float64, copy=True)
    k_out = np.zeros_like(k_in)
    v_out = np.zeros_like(v_in)
    for b in range(len(state_slot)):
        t0, t1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        s = int(state_slot[b])
        for which, src, dst in ((0, k_in, k_out), (1, v_in, v_out)):
            y, st = sconv_sequence(src[t0:t1], conv_w[which], new_state[s, which])
            dst[t0:t1] = y
            new_state[s, which] = st
    return k_out, v_out, new_state
