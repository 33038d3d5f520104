"""GPU parity of inkattn_sconv (short convolution fused with the paged
KV-cache write and the three-token state update) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuCase, assert_close, host, oracle_sconv

pytestmark = pytest.mark.gpu


def _check(case, gc, k_out, v_out, new_state):
    """Cache rows at the new tokens' slots and the state, vs the oracle."""
    from attention_sconv_amd import kvcache
    H = case.num_kv_heads
    k, v = kvcache.slots_of(gc.k_cache, gc.v_cache, case.slot_mapping.astype(np.int64))
    kg = host(k).reshape(case.num_tokens, H * 128)
    vg = host(v).reshape(case.num_tokens, H * 128)
    if case.dtype == "fp32":
        assert_close(kg, k_out, 1e-5, "k")
        assert_close(vg, v_out, 1e-5, "v")
    else:
        # one bf16 rounding (2^-9 relative) of an fp32 sum
        for g, w, nm in ((kg, k_out, "k"), (vg, v_out, "v")):
            err = np.abs(g - w)
            assert np.isfinite(g).all()
            assert (err <= np.abs(w) * 2.0 ** -8 + 1e-5).all(), f"{nm}: {err.max()}"
    # the state holds copies of pre-convolution inputs: bit-exact
    np.testing.assert_array_equal(host(gc.conv_state), new_state)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sconv_tiny_fresh_sequence(dtype):
    wl = synth.WORKLOADS["tiny_fp32_swa_prefill"]
    case = synth.make_case(dtype, [256], [0], 4, 1, wl.window, wl.bias_len, seed=0)
    gc = GpuCase(case)
    gc.sconv()
    torch.cuda.synchronize()
    _check(case, gc, *oracle_sconv(case))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sconv_ragged_batch_with_context(dtype):
    q_lens = [1, 2, 3, 17, 130, 300, 16, 33]
    ctx = [0, 5, 0, 2, 127, 1000, 1, 3]
    case = synth.make_case(dtype, q_lens, ctx, 8, 4, 0, 16, seed=1, extra_blocks=3,
                           shuffle_state_slots=True)
    gc = GpuCase(case)
    gc.sconv()
    torch.cuda.synchronize()
    _check(case, gc, *oracle_sconv(case))


def test_sconv_chunked_calls_equal_one_call():
    # Two calls (tokens split at an arbitrary point, state carried on the GPU)
    # produce bit-identical cache contents and state to a single call.
    case = synth.make_case("bf16", [77], [0], 8, 4, 0, 16, seed=2)
    one = GpuCase(case, fill_nan=False)
    one.sconv()
    two = GpuCase(case, fill_nan=False)
    import attention_sconv_amd as ink
    for a, b in ((0, 30), (30, 31), (31, 77)):
        cu = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        ink.inkattn_sconv(ink.BF16, 4, 128, 1, b - a, b - a, two.k_pre[a:b].contiguous(),
                          two.v_pre[a:b].contiguous(), two.conv_w, two.conv_state,
                          two.state_slot, cu, two.slot_mapping[a:b].contiguous(),
                          two.k_cache, two.v_cache)
    torch.cuda.synchronize()
    assert torch.equal(one.k_cache, two.k_cache)
    assert torch.equal(one.v_cache, two.v_cache)
    assert torch.equal(one.conv_state, two.conv_state)


def test_sconv_decode_batch_full_size():
    # One new token for each of 64 sequences of the 16K sliding-window decode
    # workload, with a random three-token state.
    wl = synth.WORKLOADS["swa_decode_16k"]
    case = synth.make_case("bf16", [1] * 64, [wl.seq_len - 1] * 64, 32, 4, wl.window,
                           wl.bias_len, seed=3, past_device="cuda")
    gc = GpuCase(case, fill_nan=False)
    gc.sconv()
    torch.cuda.synchronize()
    _check(case, gc, *oracle_sconv(case))


def test_sconv_delta_taps_copy_input():
    # Taps (0,0,0,1): the cache receives the input bit for bit.
    case = synth.make_case("bf16", [40, 9], [0, 0], 8, 4, 0, 16, seed=4)
    case.conv_w[:] = 0.0
    case.conv_w[:, :, 3] = 1.0
    gc = GpuCase(case)
    gc.sconv()
    torch.cuda.synchronize()
    from attention_sconv_amd import kvcache
    k, v = kvcache.slots_of(gc.k_cache, gc.v_cache, case.slot_mapping.astype(np.int64))
    np.testing.assert_array_equal(host(k).reshape(49, 512), case.k_pre)
    np.testing.assert_array_equal(host(v).reshape(49, 512), case.v_pre)
