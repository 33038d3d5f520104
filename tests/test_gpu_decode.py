"""GPU parity of inkattn_relattn_decode (split-K paged decode + LSE merge),
run after inkattn_sconv has written the new token, against the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (GpuCase, assert_attention, assert_close, assert_lse, assert_parity, host,
                      oracle_kv, oracle_sconv)

pytestmark = pytest.mark.gpu


def _expected(case, seqs=None, lo_window=True):
    k_new, v_new, _ = oracle_sconv(case)
    G = case.num_q_heads // case.num_kv_heads
    outs, lses = [], []
    for b in (range(len(case.q_lens)) if seqs is None else seqs):
        L = int(case.seq_lens[b])
        lo = max(0, L - case.window) if (case.window and lo_window) else 0
        K, V = oracle_kv(case, b, k_new, v_new, lo=lo)
        o, l = oracle.relattn_decode(case.q[b], K, V, case.bias, case.window, G)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def _run_and_check(case, num_splits=0, seqs=None, scale_aware=False):
    gc = GpuCase(case)
    gc.sconv()
    out, lse = gc.decode(num_splits)
    torch.cuda.synchronize()
    want_o, want_l = _expected(case, seqs)
    sel = list(range(len(case.q_lens))) if seqs is None else list(seqs)
    errs = assert_attention(host(out)[sel], want_o, host(lse)[sel], want_l, case.dtype,
                            "decode", scale_aware)
    return gc, out, lse, errs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4), (16, 1), (8, 8)])
@pytest.mark.parametrize("W,R", [(0, 5000), (64, 64), (300, 40)])
def test_decode_ragged_lengths(dtype, Hq, Hkv, W, R):
    # lengths cover a single key, page edges and unaligned tails
    L = [1, 2, 127, 128, 129, 1000, 4097]
    case = synth.make_case(dtype, [1] * len(L), [x - 1 for x in L], Hq, Hkv, W, R,
                           seed=10 + Hq + W, extra_blocks=2)
    _run_and_check(case)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 40])
def test_decode_split_counts(num_splits):
    case = synth.make_case("fp32", [1] * 3, [2999, 5000, 640], 32, 4, 0, 6000, seed=20)
    _run_and_check(case, num_splits)


def test_decode_split_invariance_and_determinism():
    case = synth.make_case("fp32", [1] * 4, [4095, 4096, 333, 9000], 32, 4, 2048, 2048,
                           seed=21)
    gc = GpuCase(case)
    gc.sconv()
    o1, l1 = gc.decode(1)
    o5, l5 = gc.decode(5)
    o5b, l5b = gc.decode(5)
    torch.cuda.synchronize()
    assert torch.equal(o5, o5b) and torch.equal(l5, l5b)          # bitwise repeatable
    assert_close(host(o5), host(o1), 1e-5, "split 5 vs 1")
    assert_close(host(l5), host(l1), 1e-5, "lse split 5 vs 1")


def test_decode_constant_value_passthrough():
    # every cached and new V equal to one vector -> output is that vector
    case = synth.make_case("bf16", [1, 1], [700, 3000], 32, 4, 0, 4096, seed=22)
    vec = synth.round_bf16(np.random.default_rng(0).standard_normal(128).astype(np.float32))
    case.past_v[:] = np.tile(vec, (case.past_v.shape[0], 4, 1))
    case.v_pre[:] = np.tile(vec, 4)
    case.conv_w[1] = 0.0
    case.conv_w[1, :, 3] = 1.0
    gc = GpuCase(case)
    gc.sconv()
    out, _ = gc.decode()
    torch.cuda.synchronize()
    assert_close(host(out), np.broadcast_to(vec, (2, 32, 128)), 2 ** -8, "constant V")


def test_decode_swa_16k_full_size():
    # the 16K sliding-window decode workload, every row, auto split count
    wl = synth.WORKLOADS["swa_decode_16k"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, scale_aware=True)


def test_decode_full_1m_full_size():
    # the 1M-key full-attention decode workload, every head of all four
    # sequences, auto split count (16 splits and the LSE merge).  Outputs are
    # ~1e-2 and lse ~15 here, so the scale-aware output bound and the
    # absolute lse bound are what can see a lost or mis-weighted split.
    wl = synth.WORKLOADS["full_decode_1m"]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    _run_and_check(case, scale_aware=True)


@pytest.mark.parametrize("name,seqs", [("swa_decode_16k", None), ("full_decode_1m", [0, 3])])
def test_decode_full_size_shapes_fp32(name, seqs):
    # the 16K sliding-window and 1M full decode workloads with fp32 storage
    # (a 16 GiB cache at 1M): the same split counts and merge, held to 1e-5
    wl = dataclasses.replace(synth.WORKLOADS[name], dtype="fp32")
    case = synth.workload_case(wl, seed=4, past_device="cuda")
    _run_and_check(case, seqs=seqs)


def test_tiny_fp32_prefill_then_decode_against_oracle():
    # The tiny workload as a serving run: prefill of the first 192 tokens,
    # then 64 decode steps (sconv of the new token through the cached state,
    # then split-K decode), every output row against the oracle's attention
    # over the whole sequence.
    import attention_sconv_amd as ink
    wl = synth.WORKLOADS["tiny_fp32_swa_prefill"]
    T, P, Hq, Hkv = 256, 192, 4, 1
    case = synth.make_case("fp32", [T], [0], Hq, Hkv, wl.window, wl.bias_len, seed=0)
    k_all, v_all, _ = oracle_sconv(case)
    want, want_lse = oracle.relattn_prefill(case.q, k_all.reshape(T, Hkv, 128),
                                            v_all.reshape(T, Hkv, 128), case.bias,
                                            wl.window, Hq // Hkv)
    gc = GpuCase(case, fill_nan=True)
    d = gc.desc()
    cu = torch.tensor([0, P], dtype=torch.int32, device="cuda")
    sl = torch.tensor([P], dtype=torch.int32, device="cuda")
    ink.inkattn_sconv(ink.FP32, Hkv, 128, 1, P, P, gc.k_pre[:P].contiguous(),
                      gc.v_pre[:P].contiguous(), gc.conv_w, gc.conv_state, gc.state_slot, cu,
                      gc.slot_mapping[:P].contiguous(), gc.k_cache, gc.v_cache)
    o_p = torch.empty((P, Hq, 128), device="cuda")
    l_p = torch.empty((P, Hq), device="cuda")
    ink.inkattn_relattn_prefill(d, 1, P, P, gc.q[:P].contiguous(), gc.k_cache, gc.v_cache,
                                gc.block_table, gc.block_table.shape[1], cu, sl, gc.bias, o_p,
                                l_p)
    outs, lses = [o_p], [l_p]
    one = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    ws_bytes = ink.inkattn_relattn_decode_workspace_size(d, 1, T, 0)
    ws = torch.empty(ws_bytes // 4 + 4, device="cuda")
    for t in range(P, T):
        ink.inkattn_sconv(ink.FP32, Hkv, 128, 1, 1, 1, gc.k_pre[t:t + 1].contiguous(),
                          gc.v_pre[t:t + 1].contiguous(), gc.conv_w, gc.conv_state,
                          gc.state_slot, one, gc.slot_mapping[t:t + 1].contiguous(),
                          gc.k_cache, gc.v_cache)
        L = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        o = torch.empty((1, Hq, 128), device="cuda")
        lse = torch.empty((1, Hq), device="cuda")
        ink.inkattn_relattn_decode(d, 1, t + 1, gc.q[t:t + 1].contiguous(), gc.k_cache,
                                   gc.v_cache, gc.block_table, gc.block_table.shape[1], L,
                                   gc.bias, o, lse, 0, ws, ws_bytes)
        outs.append(o)
        lses.append(lse)
    torch.cuda.synchronize()
    assert_parity(host(torch.cat(outs)), want, "fp32", "prefill + decode outputs")
    assert_lse(host(torch.cat(lses)), want_lse, "fp32", "prefill + decode lse")


@pytest.mark.parametrize("W,R", [(1, 1), (1, 300), (129, 1)])
def test_decode_window_and_table_edges(W, R):
    # a window of only the new token, a one-entry bias table, a window one
    # key past a page
    L = [1, 128, 129, 4097]
    case = synth.make_case("bf16", [1] * len(L), [x - 1 for x in L], 32, 4, W, R,
                           seed=23 + W + R)
    _run_and_check(case)
