"""GPU parity of the FP8 (E4M3) KV cache: inkattn_sconv_fp8 writes codes of the
convolved keys and values, inkattn_relattn_decode_fp8 attends over them.

Codes: the kernel evaluates the convolution and the division by the scale in
fp32, so a code may differ from the oracle's (fp64) code only where the exact
quotient lies within that evaluation's error bound of a rounding boundary;
there either neighbour is a correct rounding.  Attention: the oracle attends
over the read-back values of the cached context's codes and of its own codes
for the new tokens, at the bf16 bound.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from attention_sconv_amd import kvcache
from gpu_util import (GpuCase, assert_attention, assert_close, fp8_codes, host, oracle_kv,
                      oracle_sconv)

pytestmark = pytest.mark.gpu


def _abs_sconv(case):
    """sum_k |w_k| |x_k| per output (the scale of the fp32 rounding error)."""
    a = np.abs
    return oracle.sconv_batch(a(case.k_pre), a(case.v_pre), a(case.conv_w), a(case.conv_state),
                              case.state_slot, case.cu_seqlens)


def _check_codes(got, y, y_abs, scale, what):
    """got: uint8 codes; y: exact outputs (fp64); y_abs: sum of |terms|."""
    x = y / scale
    # fp32: three roundings in the 4-term sum (each <= 2^-24 of sum |terms|),
    # one in the product with the rounded reciprocal of the scale (and that
    # reciprocal's own rounding); bounds taken with a factor 2 to spare.
    delta = (y_abs * 2.0 ** -21 + np.abs(y) * 2.0 ** -22) / scale
    want = oracle.fp8.quantize(y, scale)
    lo = oracle.fp8.e4m3_code(x - delta)
    hi = oracle.fp8.e4m3_code(x + delta)
    ok = (got == want) | (got == lo) | (got == hi)
    bad = np.nonzero(~ok.reshape(-1))[0]
    assert len(bad) == 0, (f"{what}: {len(bad)} codes off, first at {bad[0]}: got "
                           f"{got.reshape(-1)[bad[0]]:#x} want {want.reshape(-1)[bad[0]]:#x} "
                           f"(x = {x.reshape(-1)[bad[0]]!r})")
    assert (got != want).mean() < 1e-3, f"{what}: too many boundary cases"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scales", [(1 / 32, 1 / 16), (0.0173, 0.051), (1e-3, 2e-3)])
def test_sconv_fp8_codes(dtype, scales):
    # chunks across the 8-token thread chunk and page edges, fresh and with
    # context; the last scales saturate most outputs at +-448
    q_lens = [1, 7, 8, 9, 100, 130]
    ctx = [0, 5, 0, 130, 3, 0]
    case = synth.make_case(dtype, q_lens, ctx, 8, 4, 0, 10, seed=80, extra_blocks=1)
    gc = GpuCase(case, fp8_scales=scales)
    gc.sconv()
    torch.cuda.synchronize()
    k_new, v_new, st = oracle_sconv(case)
    k_abs, v_abs, _ = _abs_sconv(case)
    kc, vc = kvcache.slots_of(gc.k_cache, gc.v_cache, case.slot_mapping)
    N = case.num_tokens
    _check_codes(kc.cpu().numpy().reshape(N, -1), k_new, k_abs, scales[0], "K")
    _check_codes(vc.cpu().numpy().reshape(N, -1), v_new, v_abs, scales[1], "V")
    # the sconv state is the same copy as with a bf16 / fp32 cache
    assert np.array_equal(host(gc.conv_state), st)


def _expected(case, gc, seqs=None):
    ks, vs = gc.fp8
    k_new, v_new, _ = oracle_sconv(case)
    G = case.num_q_heads // case.num_kv_heads
    outs, lses = [], []
    for b in (range(len(case.q_lens)) if seqs is None else seqs):
        L, n = int(case.seq_lens[b]), int(case.q_lens[b])
        lo = max(0, L - n - case.window + 1) if case.window else 0
        K, V = oracle_kv(case, b, k_new, v_new, lo=lo, fp8=(gc, ks, vs))
        t0 = int(case.cu_seqlens[b])
        o, l = oracle.relattn_prefill(case.q[t0:t0 + n], K, V, case.bias, case.window, G)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def _run_and_check(case, scales, num_splits=0, seqs=None, scale_aware=False):
    gc = GpuCase(case, fp8_scales=scales)
    gc.sconv()
    out, lse = gc.decode_fp8(num_splits)
    torch.cuda.synchronize()
    want_o, want_l = _expected(case, gc, seqs)
    if seqs is None:
        rows = np.arange(case.num_tokens)
    else:
        rows = np.concatenate([np.arange(case.cu_seqlens[b], case.cu_seqlens[b + 1])
                               for b in seqs])
    assert_attention(host(out)[rows], want_o, host(lse)[rows], want_l, "bf16", "decode_fp8",
                     scale_aware)
    return gc, out, lse


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4), (16, 1)])
@pytest.mark.parametrize("W,R", [(0, 5000), (64, 64), (300, 40)])
def test_decode_fp8_ragged(Hq, Hkv, W, R):
    # one token per sequence; lengths on page edges and unaligned tails
    L = [1, 2, 127, 128, 129, 1000, 4097]
    case = synth.make_case("bf16", [1] * len(L), [x - 1 for x in L], Hq, Hkv, W, R,
                           seed=90 + Hq + W, extra_blocks=2)
    _run_and_check(case, (1 / 64, 1 / 32))


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (16, 1)])
def test_decode_fp8_multi_query(Hq, Hkv):
    # MTP verification over an FP8 cache: 1..9 tokens per sequence (several
    # column tiles per work-group), plus the largest query count
    q_lens = [1, 2, 9, 5, 3, 9, 16]
    ctx = [0, 126, 119, 1000, 3, 4090, 250]
    case = synth.make_case("bf16", q_lens, ctx, Hq, Hkv, 512, 512, seed=91 + Hq)
    _run_and_check(case, (0.02, 0.03))


@pytest.mark.parametrize("num_splits", [1, 3, 40])
def test_decode_fp8_split_counts(num_splits):
    case = synth.make_case("bf16", [1, 4, 1], [2999, 5000, 640], 32, 4, 0, 6000, seed=92)
    _run_and_check(case, (1 / 64, 1 / 64), num_splits)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 40])
def test_decode_fp8_one_token_split_counts(num_splits):
    # one token per sequence and 8 heads per group: one column tile, 64-key
    # items (a split's range can end on either half of a page); 40 splits
    # leave splits of the shorter sequences without a page
    case = synth.make_case("bf16", [1, 1, 1, 1], [2999, 5000, 640, 63], 32, 4, 0, 6000,
                           seed=94)
    _run_and_check(case, (1 / 64, 1 / 32), num_splits)


def test_decode_fp8_equals_bf16_cache_of_the_same_values():
    # With power-of-two scales every read-back value is a bf16, so a bf16
    # cache can hold exactly the same keys and values: the two decodes differ
    # only in the order of the fp32 sums.
    case = synth.make_case("bf16", [1, 3, 1, 9], [4095, 700, 17, 3000], 32, 4, 2048, 2048,
                           seed=93)
    ks, vs = 1 / 64, 1 / 32
    g8 = GpuCase(case, fill_nan=False, fp8_scales=(ks, vs))
    g8.sconv()
    gb = GpuCase(case, fill_nan=False)
    kf = g8.k_cache.view(torch.float8_e4m3fn).float() * ks
    vf = g8.v_cache.view(torch.float8_e4m3fn).float() * vs
    torch.cuda.synchronize()
    gb.k_cache = kf.to(torch.bfloat16).contiguous()
    gb.v_cache = vf.to(torch.bfloat16).contiguous()
    assert torch.equal(gb.k_cache.float(), kf) and torch.equal(gb.v_cache.float(), vf)
    o8, l8 = g8.decode_fp8()
    ob, lb = gb.decode_mq()
    o8b, l8b = g8.decode_fp8()
    torch.cuda.synchronize()
    assert torch.equal(o8, o8b) and torch.equal(l8, l8b)          # repeatable
    assert_close(host(o8), host(ob), 1e-2, "fp8 vs bf16 cache", relative=True)
    assert_close(host(l8), host(lb), 1e-4, "lse fp8 vs bf16 cache")


@pytest.mark.parametrize("W,R", [(1, 1), (2, 7), (257, 3000)])
def test_decode_fp8_window_edges(W, R):
    case = synth.make_case("bf16", [1, 9, 4, 1], [0, 300, 128, 4000], 32, 4, W, R,
                           seed=94 + W)
    _run_and_check(case, (1 / 16, 1 / 16))


def test_decode_fp8_swa_16k_full_size():
    # the 16K sliding-window decode workload with an FP8 cache, every row
    wl = synth.WORKLOADS["swa_decode_16k"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, (1 / 64, 1 / 64), scale_aware=True)


def test_decode_fp8_full_1m_full_size():
    # the 1M-key full-attention decode workload over an E4M3 cache (half the
    # 8 GiB of the bf16 cache), every head of all four sequences, auto split
    # count and the LSE merge
    wl = synth.WORKLOADS["full_decode_1m"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, (1 / 64, 1 / 64), scale_aware=True)


@pytest.mark.parametrize("Hq,Hkv,q_max", [(32, 4, 5), (32, 4, 8), (4, 1, 9), (32, 4, 9)])
@pytest.mark.parametrize("W,R", [(0, 3000), (2048, 2048)])
def test_decode_fp8_multi_query_column_tiles(Hq, Hkv, q_max, W, R):
    # 3, 4, 3 and 5 column tiles of 16 (token, head) columns, the register-
    # resident multi-query kernel over an E4M3 cache; contexts end on and off
    # page edges and on every quarter of a page
    q_lens = [q_max, 1, q_max - 1, 2, q_max]
    ctx = [2048, 127, 4000 - q_max, 31, 96]
    case = synth.make_case("bf16", q_lens, ctx, Hq, Hkv, W, R, seed=97 + Hq + q_max + W)
    _run_and_check(case, (1 / 32, 1 / 64))


def test_decode_fp8_multi_query_long_bias_table():
    # R = 2^22 with 8 q-heads (2^25 bias entries, row starts past 2^24), the
    # register-resident multi-query kernel over an E4M3 cache
    case = synth.make_case("bf16", [9, 4, 9], [3000, 130, 1000], 8, 1, 0, 1 << 22, seed=98)
    _run_and_check(case, (1 / 32, 1 / 64))


def test_decode_fp8_mtp9_16k_sampled():
    # the 16K sliding-window verification workload (64 sequences x 9 query
    # tokens) over an E4M3 cache at full size; the oracle checks every token
    # and head of 8 sequences spread over the batch
    wl = synth.WORKLOADS["swa_decode_16k_mtp9"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, (1 / 64, 1 / 64), seqs=list(range(0, wl.batch, 9)) + [wl.batch - 1],
                   scale_aware=True)


@pytest.mark.parametrize("peak", [15.0, 50.0])
def test_decode_fp8_multi_query_old_keys_far_above_the_newest(peak):
    # as in the bf16-cache test: keys 1000 or more positions back get `peak`
    # added to their logits and are met last, so the register kernel's
    # softmax reference is passed by 22 or 72 (log2 units), the second
    # through a rerun from the exact column max
    case = synth.make_case("bf16", [9, 3, 9], [3000, 1100, 1500], 32, 4, 0, 2048, seed=98)
    case.bias[:, 1000:] = synth.round_bf16(case.bias[:, 1000:] + np.float32(peak))
    _run_and_check(case, (1 / 32, 1 / 32))


def _run_prefill_and_check(case, scales):
    gc = GpuCase(case, fp8_scales=scales)
    gc.sconv()
    out, lse = gc.prefill_fp8()
    torch.cuda.synchronize()
    want_o, want_l = _expected(case, gc)
    assert_attention(host(out), want_o, host(lse), want_l, "bf16", "prefill_fp8")
    return gc, out, lse


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4)])
@pytest.mark.parametrize("W,R", [(0, 3000), (64, 64), (300, 40)])
def test_prefill_fp8_chunks_after_context(Hq, Hkv, W, R):
    # chunks of 1 .. 300 tokens after contexts that end on and off page edges
    q_lens = [300, 1, 77, 129, 5]
    ctx = [0, 127, 700, 256, 1500]
    case = synth.make_case("bf16", q_lens, ctx, Hq, Hkv, W, R, seed=95 + Hq + W,
                           extra_blocks=2)
    _run_prefill_and_check(case, (1 / 64, 1 / 32))


@pytest.mark.parametrize("scales", [(0.0173, 0.051), (2.0, 0.5)])
def test_prefill_fp8_scales(scales):
    case = synth.make_case("bf16", [200, 64], [900, 0], 32, 4, 512, 512, seed=96)
    _run_prefill_and_check(case, scales)


def test_prefill_fp8_matches_decode_fp8():
    # the same query tokens through the E4M3 prefill and the E4M3 multi-query
    # decode: two kernels, one definition
    case = synth.make_case("bf16", [9, 3, 16], [4000, 127, 700], 32, 4, 2048, 2048, seed=97)
    gc = GpuCase(case, fp8_scales=(1 / 64, 1 / 32))
    gc.sconv()
    op, lp = gc.prefill_fp8()
    od, ld = gc.decode_fp8()
    op2, lp2 = gc.prefill_fp8()
    torch.cuda.synchronize()
    assert torch.equal(op, op2) and torch.equal(lp, lp2)
    assert_close(host(op), host(od), 2e-2, "prefill_fp8 vs decode_fp8")
    assert_close(host(lp), host(ld), 2e-2, "lse prefill_fp8 vs decode_fp8")


def test_prefill_fp8_empty_chunks_in_batch():
    case = synth.make_case("bf16", [0, 100, 0, 33], [50, 0, 300, 500], 32, 4, 64, 100, seed=99)
    _run_prefill_and_check(case, (1 / 64, 1 / 32))
