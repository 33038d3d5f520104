"""GPU parity of inkattn_sconv_out (the short convolution of the attention
output or the MoE output, with its three-token state) against the oracle's
per-sequence convolution."""

import numpy as np
import pytest
import torch

import attention_sconv_amd as ink
import oracle
import synth
from gpu_util import assert_parity, ddtype, dev, host, idev

pytestmark = pytest.mark.gpu


def _run(case, x=None, state=None, stream=None):
    """One call on device copies; returns (y, state) device tensors."""
    C = case.x.shape[1]
    xd = dev(case.x if x is None else x, case.dtype)
    st = dev(case.conv_state, case.dtype) if state is None else state
    y = torch.full_like(xd, float("nan"))
    ink.inkattn_sconv_out(ddtype(case.dtype), C, len(case.q_lens), xd.shape[0],
                          int(case.q_lens.max(initial=0)), xd, dev(case.conv_w, case.dtype),
                          st, idev(case.state_slot), idev(case.cu_seqlens), y, stream)
    return y, st


def _expected(case, x=None, state=None):
    x = case.x if x is None else x
    state = np.array(case.conv_state if state is None else state, dtype=np.float64)
    y = np.zeros(x.shape)
    for b in range(len(case.q_lens)):
        t0, t1 = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        s = int(case.state_slot[b])
        y[t0:t1], state[s] = oracle.sconv_sequence(x[t0:t1], case.conv_w, state[s])
    return y, state


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("C", [8, 128, 1000, 4096, 8192])
def test_sconv_out_ragged(dtype, C):
    # chunks of 1-3 tokens (the new state still holds old state rows), around
    # the 8-token thread chunk and the 32-token work-group edges
    q_lens = [1, 2, 3, 4, 7, 8, 9, 31, 32, 33, 70]
    fresh = [b % 3 == 0 for b in range(len(q_lens))]
    case = synth.make_sconv_out_case(dtype, q_lens, C, seed=C, fresh=fresh)
    y, st = _run(case)
    torch.cuda.synchronize()
    want_y, want_st = _expected(case)
    assert_parity(host(y), want_y, dtype, "y")
    # the state is a copy of input rows: exact, and rows no sequence owns stay
    assert np.array_equal(host(st), want_st)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sconv_out_chunked_equals_whole(dtype):
    # a sequence convolved in chunks of 1, 2, 5 and 40 tokens carries the state
    # across calls: same outputs and final state as one call over all of it
    C, T = 512, 48
    case = synth.make_sconv_out_case(dtype, [T], C, seed=5, extra_slots=0, fresh=[True])
    y_all, st_all = _run(case)
    st = dev(case.conv_state, dtype)
    parts = []
    t = 0
    for n in (1, 2, 5, 40):
        sub = synth.SconvOutCase(dtype=dtype, x=case.x[t:t + n], conv_w=case.conv_w,
                                 conv_state=case.conv_state, state_slot=case.state_slot,
                                 cu_seqlens=np.array([0, n]), q_lens=np.array([n]))
        y, st = _run(sub, state=st)
        parts.append(y)
        t += n
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts), y_all)
    assert torch.equal(st, st_all)
    want_y, _ = _expected(case)
    assert_parity(host(y_all), want_y, dtype, "y")


def test_sconv_out_empty_sequences_and_stream():
    # zero-length chunks leave their state alone; a side stream is honoured
    case = synth.make_sconv_out_case("bf16", [0, 5, 0, 17], 256, seed=9)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y, st = _run(case, stream=s)
    s.synchronize()
    want_y, want_st = _expected(case)
    assert_parity(host(y), want_y, "bf16", "y")
    assert np.array_equal(host(st), want_st)


def test_sconv_out_full_size():
    # 64 sequences x 512 tokens of a 4096-wide activation (a stand-in width;
    # the pages give none), bf16; the oracle checks every element
    C = 4096
    case = synth.make_sconv_out_case("bf16", [512] * 64, C, seed=11)
    y, st = _run(case)
    torch.cuda.synchronize()
    want_y, want_st = _expected(case)
    assert_parity(host(y), want_y, "bf16", "y")
    assert np.array_equal(host(st), want_st)
