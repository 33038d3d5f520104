"""inkattn_relattn_decode_noalloc (split partials in the library's static
scratch array) against inkattn_relattn_decode (partials in a workspace the
caller allocates), through the C ABI: two calls in a row on one GPU, the
second with a smaller input, each held to the parity bound of its storage
dtype (and, since both run the same kernels with the same split count,
bitwise equal)."""

import numpy as np
import pytest
import torch

import attention_sconv_amd as ink
import synth
from gpu_util import GpuCase, assert_attention, host

pytestmark = pytest.mark.gpu


def _both(case, num_splits):
    gc = GpuCase(case)
    gc.sconv()
    torch.cuda.synchronize()
    want_o, want_l = gc.decode(num_splits)
    d = gc.desc()
    B, L = len(case.q_lens), int(case.seq_lens.max())
    out = torch.full_like(gc.q, float("nan"))
    lse = torch.full((B, case.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ink.inkattn_relattn_decode_noalloc(d, B, L, gc.q, gc.k_cache, gc.v_cache, gc.block_table,
                                       gc.block_table.shape[1], gc.seq_lens, gc.bias, out, lse,
                                       num_splits)
    torch.cuda.synchronize()
    return out, lse, want_o, want_l


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_noalloc_decode_two_calls_second_smaller(dtype):
    # call 1: 4 sequences of 20-60K keys, full causal, 16 splits (the 1M
    # decode's split count): 4 x 32 x 16 partial rows in the scratch
    big = synth.make_case(dtype, [1] * 4, [20000, 61000, 33333, 47000], 32, 4, 0, 70000,
                          seed=120)
    # call 2: 3 shorter sequences, sliding window, 5 splits: fewer rows, so
    # the scratch still holds call 1's rows beyond them
    small = synth.make_case(dtype, [1] * 3, [3000, 700, 5000], 32, 4, 2048, 2048, seed=121)
    for case, splits in ((big, 16), (small, 5), (small, 0)):
        out, lse, want_o, want_l = _both(case, splits)
        assert torch.equal(out, want_o) and torch.equal(lse, want_l)
        assert_attention(host(out), host(want_o), host(lse), host(want_l), dtype,
                         f"noalloc vs workspace ({splits} splits)")


def test_noalloc_decode_one_split_and_rejection():
    # one split writes the output directly (no scratch); a request whose
    # partials exceed the scratch is refused before anything runs
    case = synth.make_case("bf16", [1] * 2, [900, 4000], 32, 4, 1024, 1024, seed=122)
    out, lse, want_o, want_l = _both(case, 1)
    assert torch.equal(out, want_o) and torch.equal(lse, want_l)
    gc = GpuCase(case)
    d = gc.desc()
    before = gc.q.clone()
    with pytest.raises(ink.InkattnError) as err:
        ink.inkattn_relattn_decode_noalloc(d, 2, 5000, gc.q, gc.k_cache, gc.v_cache,
                                           gc.block_table, gc.block_table.shape[1],
                                           gc.seq_lens, gc.bias, gc.q, None,
                                           ink.NOALLOC_SCRATCH_BYTES // (2 * 32 * 512) + 1)
    assert err.value.status == ink.ESCRATCH
    torch.cuda.synchronize()
    assert torch.equal(gc.q, before)
    assert np.isfinite(host(out)).all()
