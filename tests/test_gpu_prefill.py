"""GPU parity of inkattn_relattn_prefill (run after inkattn_sconv has written
the new tokens' keys and values) against the oracle."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuCase, assert_attention, assert_close, host, oracle_kv, oracle_sconv

pytestmark = pytest.mark.gpu


def _expected(case, rows_per_seq=None, stored_kv=False):
    """Oracle output for the chosen chunk rows of every sequence; returns
    (token indices, out [n, Hq, d], lse [n, Hq]).  With ``stored_kv`` (bf16
    cases) the oracle reads the post-convolution K/V as the cache stores them,
    rounded to bf16, instead of in fp64."""
    k_new, v_new, _ = oracle_sconv(case)
    G = case.num_q_heads // case.num_kv_heads
    toks, outs, lses = [], [], []
    for b in range(len(case.q_lens)):
        qn = int(case.q_lens[b])
        rows = np.arange(qn) if rows_per_seq is None else np.asarray(rows_per_seq(b, qn))
        t0 = int(case.cu_seqlens[b])
        K, V = oracle_kv(case, b, k_new, v_new)
        if stored_kv and case.dtype == "bf16":
            K = synth.round_bf16(K.astype(np.float32)).astype(np.float64)
            V = synth.round_bf16(V.astype(np.float32)).astype(np.float64)
        o, l = oracle.relattn_prefill(case.q[t0:t0 + qn], K, V, case.bias, case.window, G,
                                      rows=rows)
        toks.append(t0 + rows)
        outs.append(o)
        lses.append(l)
    return np.concatenate(toks), np.concatenate(outs), np.concatenate(lses)


def _run_and_check(case, rows_per_seq=None, stored_kv=False, scale_aware=False):
    gc = GpuCase(case)
    gc.sconv()
    out, lse = gc.prefill()
    torch.cuda.synchronize()
    toks, want_o, want_l = _expected(case, rows_per_seq, stored_kv)
    assert_attention(host(out)[toks], want_o, host(lse)[toks], want_l, case.dtype, "prefill",
                     scale_aware)
    return gc, out, lse


def test_prefill_tiny_fp32_workload():
    # 1 sequence, T=256, Hq=4, Hkv=1, window 64, R=64, fp32, zero sconv state
    wl = synth.WORKLOADS["tiny_fp32_swa_prefill"]
    _run_and_check(synth.workload_case(wl, seed=0))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4), (8, 8)])
@pytest.mark.parametrize("W,R", [(0, 1000), (64, 64), (200, 30)])
def test_prefill_ragged_fresh(dtype, Hq, Hkv, W, R):
    # chunk lengths around the 128-row query tile and 64-key KV tile edges
    q_lens = [1, 5, 63, 64, 65, 127, 128, 129, 300]
    case = synth.make_case(dtype, q_lens, [0] * len(q_lens), Hq, Hkv, W, R,
                           seed=30 + Hq + W, extra_blocks=2)
    _run_and_check(case)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("W", [0, 100])
def test_prefill_chunk_after_context(dtype, W):
    # chunked prefill: new tokens follow cached context (random past K/V and
    # sconv state), chunk at the bottom-right of the causal mask
    q_lens = [1, 70, 129, 256, 33]
    ctx = [5, 200, 1000, 64, 3]
    case = synth.make_case(dtype, q_lens, ctx, 32, 4, W, 300, seed=40 + W)
    _run_and_check(case)


def test_prefill_decode_consistency_on_gpu():
    # prefill of all T tokens == prefill of the first P + T-P decode steps
    # (sconv state and paged cache carried on the GPU).
    T, P = 200, 150
    case = synth.make_case("fp32", [T], [0], 16, 2, 64, 100, seed=50)
    full = GpuCase(case, fill_nan=False)
    full.sconv()
    o_full, l_full = full.prefill()
    import attention_sconv_amd as ink
    inc = GpuCase(case, fill_nan=False)
    d = inc.desc()
    cu = torch.tensor([0, P], dtype=torch.int32, device="cuda")
    sl = torch.tensor([P], dtype=torch.int32, device="cuda")
    ink.inkattn_sconv(ink.FP32, 2, 128, 1, P, P, inc.k_pre[:P].contiguous(),
                      inc.v_pre[:P].contiguous(), inc.conv_w, inc.conv_state, inc.state_slot,
                      cu, inc.slot_mapping[:P].contiguous(), inc.k_cache, inc.v_cache)
    o_p = torch.empty((P, 16, 128), device="cuda")
    ink.inkattn_relattn_prefill(d, 1, P, P, inc.q[:P].contiguous(), inc.k_cache,
                                inc.v_cache, inc.block_table, inc.block_table.shape[1], cu, sl,
                                inc.bias, o_p, None)
    outs = [o_p]
    one = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    ws_bytes = ink.inkattn_relattn_decode_workspace_size(d, 1, T, 0)
    ws = torch.empty(ws_bytes // 4 + 4, device="cuda")
    for t in range(P, T):
        ink.inkattn_sconv(ink.FP32, 2, 128, 1, 1, 1, inc.k_pre[t:t + 1].contiguous(),
                          inc.v_pre[t:t + 1].contiguous(), inc.conv_w, inc.conv_state,
                          inc.state_slot, one, inc.slot_mapping[t:t + 1].contiguous(),
                          inc.k_cache, inc.v_cache)
        L = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        o = torch.empty((1, 16, 128), device="cuda")
        ink.inkattn_relattn_decode(d, 1, t + 1, inc.q[t:t + 1].contiguous(), inc.k_cache,
                                   inc.v_cache, inc.block_table, inc.block_table.shape[1], L,
                                   inc.bias, o, None, 0, ws, ws_bytes)
        outs.append(o)
    torch.cuda.synchronize()
    assert_close(host(torch.cat(outs)), host(o_full), 1e-5, "incremental vs one-shot")
    assert torch.equal(inc.conv_state, full.conv_state)


def test_prefill_deterministic_and_block_placement_invariant():
    case = synth.make_case("bf16", [300, 77], [0, 0], 32, 4, 0, 400, seed=60, extra_blocks=5)
    gc = GpuCase(case, fill_nan=False)
    gc.sconv()
    o1, l1 = gc.prefill()
    o2, l2 = gc.prefill()
    # move every page to another physical block and rewrite the table
    perm = torch.randperm(case.num_blocks, generator=torch.Generator().manual_seed(1))
    perm_d = perm.to("cuda")
    k2 = torch.empty_like(gc.k_cache)
    v2 = torch.empty_like(gc.v_cache)
    k2[perm_d] = gc.k_cache
    v2[perm_d] = gc.v_cache
    gc.k_cache, gc.v_cache = k2, v2
    gc.block_table = perm_d.to(torch.int32)[gc.block_table.long()].contiguous()
    o3, l3 = gc.prefill()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def _late_rows(q_len, n, seed):
    """About n distinct rows of a chunk: tile and window edges, the last 64
    rows, and random rows whose density grows toward the end of the chunk
    (late rows attend the most keys, so their outputs are the smallest)."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 3, 63, 64, 127, 128, 129, 255, 256, 257, 2047, 2048, 2049, 4095, 4096,
             q_len // 2, q_len - 257, q_len - 256, q_len - 129, q_len - 128]
    rows = set(r for r in fixed if 0 <= r < q_len)
    rows.update(range(max(0, q_len - 64), q_len))
    while len(rows) < min(n, q_len):
        u = rng.random(n)
        rows.update((q_len - 1 - np.floor(q_len * u * u)).astype(np.int64).tolist())
    return np.array(sorted(rows))


def test_prefill_swa_8k_full_size():
    # batch 1, T=8192, Hq=32, Hkv=4, window 2048, R=2048, bf16: every row of
    # every head against the oracle, with the scale-aware bound as well
    wl = synth.WORKLOADS["swa_prefill_8k"]
    case = synth.workload_case(wl, seed=0)
    _run_and_check(case, scale_aware=True)


def test_prefill_full_32k_full_size_sampled():
    # batch 2, T=32768, full causal, R=32768, bf16: 512 rows per sequence,
    # weighted toward the late rows (up to 32K keys, outputs ~0.04), all heads
    wl = synth.WORKLOADS["full_prefill_32k"]
    case = synth.workload_case(wl, seed=0)
    _run_and_check(case, rows_per_seq=lambda b, n: _late_rows(n, 512, 7 + b), scale_aware=True)


@pytest.mark.parametrize("name,rows", [("swa_prefill_8k", 256), ("full_prefill_32k", 128)])
def test_prefill_full_size_shapes_fp32(name, rows):
    # the 8K sliding-window and 32K full-causal workloads with fp32 storage:
    # the same tiling, splits of work and merges as bf16, held to 1e-5
    wl = dataclasses.replace(synth.WORKLOADS[name], dtype="fp32")
    case = synth.workload_case(wl, seed=3)
    _run_and_check(case, rows_per_seq=lambda b, n: _late_rows(n, rows, 11 + b))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(16, 1), (32, 4)])
@pytest.mark.parametrize("W,R", [(1, 1), (1, 50), (2, 1), (256, 1), (257, 3000), (100000, 64)])
def test_prefill_window_and_table_edges(dtype, Hq, Hkv, W, R):
    # a window of one key (only the diagonal), a bias table of one entry (a
    # constant per head), windows at and just past the 256-row query tile, and
    # a window longer than every sequence; queries span several query tiles.
    # With a window of two keys an output is a two-point interpolation whose
    # weight moves with the rounding of the stored keys by more than the bf16
    # bound allows, so the bf16 cases compare against the oracle on the keys
    # and values as the cache stores them (rounded to bf16).
    q_lens = [1, 2, 255, 256, 257, 600]
    ctx = [0, 3, 0, 130, 7, 0]
    case = synth.make_case(dtype, q_lens, ctx, Hq, Hkv, W, R, seed=70 + W % 97 + R % 13,
                           extra_blocks=1)
    _run_and_check(case, stored_kv=True)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prefill_empty_chunks_in_batch(dtype):
    # sequences with no new token in the batch: nothing of theirs is computed
    # or written, and their sconv state stays as it was
    case = synth.make_case(dtype, [0, 100, 0, 33], [50, 0, 300, 500], 32, 4, 64, 100, seed=98)
    gc, out, lse = _run_and_check(case)
    st = host(gc.conv_state)
    for b in (0, 2):
        slot = int(case.state_slot[b])
        assert np.array_equal(st[slot], case.conv_state[slot])
