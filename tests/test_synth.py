"""The seeded input module: determinism, bf16 rounding and paging bookkeeping."""

import numpy as np
import torch

import synth


def test_round_bf16_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]   # exact ties + denormal
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(synth.round_bf16(x), ref)


def test_case_is_deterministic_and_well_formed():
    a = synth.make_case("bf16", [5, 130, 1], [0, 0, 300], 8, 2, 16, 40, seed=3,
                        extra_blocks=4)
    b = synth.make_case("bf16", [5, 130, 1], [0, 0, 300], 8, 2, 16, 40, seed=3,
                        extra_blocks=4)
    for name in ("q", "k_pre", "v_pre", "conv_w", "bias", "conv_state", "block_table",
                 "slot_mapping", "past_k"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    # bf16-representable values
    np.testing.assert_array_equal(synth.round_bf16(a.q), a.q)
    # the block table hands out distinct physical blocks
    used = np.concatenate([a.block_table[i, :(a.seq_lens[i] + 127) // 128]
                           for i in range(3)])
    assert len(set(used.tolist())) == len(used)
    assert used.max() < a.num_blocks
    # slot mapping places each new token at its logical position
    pos = np.arange(300, 301)
    assert a.slot_mapping[-1] == a.block_table[2, pos[0] // 128] * 128 + pos[0] % 128
    # fresh sequences have a zero sconv state, continued ones a random one
    assert not a.conv_state[0].any() and not a.conv_state[1].any()
    assert a.conv_state[2].any()


def test_workloads_shapes():
    wl = synth.WORKLOADS["swa_decode_16k"]
    assert (wl.batch, wl.seq_len, wl.window, wl.bias_len) == (64, 16384, 4096, 4096)
    wl = synth.WORKLOADS["full_decode_1m"]
    assert wl.seq_len == 1 << 20 and wl.bias_len == 1 << 20
