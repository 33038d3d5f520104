"""GPU parity of inkattn_relattn_decode_mq: several query tokens per
sequence (the verification of multi-token-prediction drafts), run after
inkattn_sconv has written them, against the oracle's attention of those
tokens with the sequence's earlier tokens as context."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuCase, assert_attention, assert_close, host, oracle_kv, oracle_sconv

pytestmark = pytest.mark.gpu


def _expected(case, seqs=None):
    k_new, v_new, _ = oracle_sconv(case)
    G = case.num_q_heads // case.num_kv_heads
    outs, lses = [], []
    for b in (range(len(case.q_lens)) if seqs is None else seqs):
        L, n = int(case.seq_lens[b]), int(case.q_lens[b])
        lo = max(0, L - n - case.window + 1) if case.window else 0
        K, V = oracle_kv(case, b, k_new, v_new, lo=lo)
        t0 = int(case.cu_seqlens[b])
        o, l = oracle.relattn_prefill(case.q[t0:t0 + n], K, V, case.bias, case.window, G)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def _run_and_check(case, num_splits=0, seqs=None, scale_aware=False):
    gc = GpuCase(case)
    gc.sconv()
    out, lse = gc.decode_mq(num_splits)
    torch.cuda.synchronize()
    want_o, want_l = _expected(case, seqs)
    if seqs is None:
        got_o, got_l = host(out), host(lse)
    else:
        rows = np.concatenate([np.arange(case.cu_seqlens[b], case.cu_seqlens[b + 1])
                               for b in seqs])
        got_o, got_l = host(out)[rows], host(lse)[rows]
    assert_attention(got_o, want_o, got_l, want_l, case.dtype, "decode_mq", scale_aware)
    return gc, out, lse


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4), (16, 1), (8, 4)])
@pytest.mark.parametrize("W,R", [(0, 5000), (64, 64), (300, 40)])
def test_decode_mq_ragged(dtype, Hq, Hkv, W, R):
    # 1..9 query tokens (one accepted token and up to 8 drafts) on contexts
    # that put the tokens across page edges and on unaligned tails
    q_lens = [1, 2, 9, 5, 3, 9, 7]
    ctx = [0, 126, 119, 1000, 3, 4090, 250]
    case = synth.make_case(dtype, q_lens, ctx, Hq, Hkv, W, R, seed=40 + Hq + W,
                           extra_blocks=2)
    _run_and_check(case)


@pytest.mark.parametrize("num_splits", [1, 2, 5, 40])
def test_decode_mq_split_counts(num_splits):
    case = synth.make_case("fp32", [4, 9, 1], [2999, 5000, 640], 32, 4, 0, 6000, seed=41)
    _run_and_check(case, num_splits)


@pytest.mark.parametrize("num_splits", [1, 2, 5, 40])
def test_decode_mq_split_counts_bf16(num_splits):
    # 2, 5 and 1 column tiles in one call; splits that end mid-range and
    # splits that own no page (40 > pages in range) go through the merge
    case = synth.make_case("bf16", [4, 9, 1], [2999, 5000, 640], 32, 4, 0, 6000, seed=46)
    _run_and_check(case, num_splits)


def test_decode_mq_bf16_repeatable_across_calls():
    case = synth.make_case("bf16", [9, 3, 7, 9], [4000, 127, 70, 9000], 32, 4, 2048, 2048,
                           seed=47)
    gc = GpuCase(case)
    gc.sconv()
    o1, l1 = gc.decode_mq(3)
    o2, l2 = gc.decode_mq(3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_mq_swa_16k_mtp9_sampled():
    # the 16K sliding-window verification workload at full size (64 sequences
    # x 9 query tokens, auto split count); the oracle checks every token and
    # head of 8 sequences spread over the batch
    wl = synth.WORKLOADS["swa_decode_16k_mtp9"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, seqs=list(range(0, wl.batch, 9)) + [wl.batch - 1], scale_aware=True)


def test_decode_mq_sixteen_tokens():
    # the largest supported query count: 8 heads x 16 tokens = 8 column tiles
    case = synth.make_case("bf16", [16, 16, 11], [130, 2000, 0], 32, 4, 512, 512, seed=42)
    _run_and_check(case)


def test_decode_mq_one_token_matches_decode_bitwise():
    case = synth.make_case("bf16", [1] * 5, [4095, 4096, 333, 9000, 17], 32, 4, 2048, 2048,
                           seed=43)
    gc = GpuCase(case)
    gc.sconv()
    o1, l1 = gc.decode()
    o2, l2 = gc.decode_mq()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_mq_matches_prefill_and_is_repeatable():
    # the same tokens through the prefill kernel (chunk with context)
    case = synth.make_case("fp32", [6, 2, 9], [700, 4100, 1500], 32, 4, 1024, 1024, seed=44)
    gc = GpuCase(case)
    gc.sconv()
    om, lm = gc.decode_mq(3)
    om2, lm2 = gc.decode_mq(3)
    op, lp = gc.prefill()
    torch.cuda.synchronize()
    assert torch.equal(om, om2) and torch.equal(lm, lm2)
    assert_close(host(om), host(op), 1e-5, "decode_mq vs prefill")
    assert_close(host(lm), host(lp), 1e-5, "lse decode_mq vs prefill")


@pytest.mark.parametrize("W,R", [(1, 1), (2, 7), (9, 1)])
def test_decode_mq_small_windows(W, R):
    # windows shorter than the run of query tokens: early tokens' keys drop out
    # of later tokens' windows inside the same call
    case = synth.make_case("bf16", [9, 9, 4], [0, 300, 128], 32, 4, W, R, seed=45 + W)
    _run_and_check(case)


@pytest.mark.parametrize("peak", [15.0, 50.0])
@pytest.mark.parametrize("q_lens", [[9, 3, 9], [16, 12, 16]])
def test_decode_mq_old_keys_far_above_the_newest(peak, q_lens):
    # keys 1000 or more positions back get `peak` added to every logit, and
    # the kernels meet them last (pages are taken newest first): the running
    # softmax reference set by the first keys is then passed by 15 (22 in
    # log2 units: probabilities far above 1) or by 50 (72 in log2 units: the
    # register kernel recomputes its range from the exact column max).  9
    # tokens x 8 heads run the register kernel, 16 the LDS-staged one.
    case = synth.make_case("bf16", q_lens, [3000, 1100, 1500], 32, 4, 0, 2048, seed=48)
    case.bias[:, 1000:] = synth.round_bf16(case.bias[:, 1000:] + np.float32(peak))
    _run_and_check(case)


@pytest.mark.parametrize("Hq,Hkv,q_max", [(32, 4, 8), (32, 4, 6), (8, 4, 16), (4, 1, 16)])
def test_decode_mq_register_kernel_column_tiles(Hq, Hkv, q_max):
    # 4, 3, 2 and 4 column tiles of 16 (token, head) columns; contexts end on
    # and off page edges and on every quarter of a page
    q_lens = [q_max, 1, q_max - 1, 3, q_max]
    ctx = [2048, 127, 4000 - q_max, 31, 96]
    case = synth.make_case("bf16", q_lens, ctx, Hq, Hkv, 1024, 1024, seed=49 + Hq + q_max)
    _run_and_check(case)


def test_decode_mq_register_kernel_long_bias_table():
    # R = 2^22 with 8 q-heads: 2^25 bias entries, so row starts lie past 2^24
    # (full-attention layers verifying 9 tokens at a long context window)
    q_lens = [9, 4, 9]
    ctx = [3000, 130, 1000]
    case = synth.make_case("bf16", q_lens, ctx, 8, 1, 0, 1 << 22, seed=53)
    _run_and_check(case)
