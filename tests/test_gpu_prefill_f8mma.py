"""GPU parity of the prefill with FP8 matrix products
(``inkattn_relattn_prefill_fp8_mma``) against the oracle.

Expected values: the oracle's attention over the read-back keys and values
of the E4M3 cache and over the queries read back from the oracle's own
per-tile quantizer (``oracle.fp8.quantize_query_tiles``, the scheme the
kernel implements).  The one rounding the oracle does not reproduce is that
of the softmax probabilities to E4M3 inside the online softmax; the oracle
bounds what it can move (``oracle.relattn_prefill_p8_bounds``), and each
case checks them with ``parity.check_p8`` (every output and lse within the
bound, and the errors' root mean square below 2 predicted spreads; the
oracle's own Monte Carlo run of the rounding gives about 0.7, and
``test_parity_checker`` shows a dropped key tile failing).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuCase, host, oracle_kv, oracle_sconv
from parity import check_p8

pytestmark = pytest.mark.gpu


def _expected(case, gc, rows=None):
    ks, vs = gc.fp8
    k_new, v_new, _ = oracle_sconv(case)
    G = case.num_q_heads // case.num_kv_heads
    qdq, _ = oracle.fp8.quantize_query_tiles(case.q, case.cu_seqlens)
    parts = []
    sel = []
    for b in range(len(case.q_lens)):
        L, n = int(case.seq_lens[b]), int(case.q_lens[b])
        if n == 0:
            continue
        lo = max(0, L - n - case.window + 1) if case.window else 0
        K, V = oracle_kv(case, b, k_new, v_new, lo=lo, fp8=(gc, ks, vs))
        t0 = int(case.cu_seqlens[b])
        r = np.arange(n) if rows is None else np.asarray(rows[b])
        parts.append(oracle.relattn_prefill_p8_bounds(qdq[t0:t0 + n], K, V, case.bias,
                                                      case.window, G, rows=r))
        sel.append(t0 + r)
    return np.concatenate(sel), [np.concatenate([p[k] for p in parts]) for k in range(6)]


def _run(case, scales, rows=None):
    gc = GpuCase(case, fp8_scales=scales)
    gc.sconv()
    out, lse = gc.prefill_fp8_mma()
    torch.cuda.synchronize()
    sel, exp = _expected(case, gc, rows)
    check_p8(host(out)[sel], host(lse)[sel], exp, "prefill_fp8_mma")
    return gc, out, lse


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (32, 4)])
@pytest.mark.parametrize("W,R", [(0, 3000), (64, 64), (300, 40)])
def test_prefill_fp8_mma_chunks_after_context(Hq, Hkv, W, R):
    # chunks of 1 .. 300 tokens after contexts that end on and off page edges
    q_lens = [300, 1, 77, 129, 5]
    ctx = [0, 127, 700, 256, 1500]
    case = synth.make_case("bf16", q_lens, ctx, Hq, Hkv, W, R, seed=195 + Hq + W,
                           extra_blocks=2)
    _run(case, (1 / 64, 1 / 32))


@pytest.mark.parametrize("scales", [(0.0173, 0.051), (2.0, 0.5)])
def test_prefill_fp8_mma_scales(scales):
    case = synth.make_case("bf16", [200, 64], [900, 0], 32, 4, 512, 512, seed=196)
    _run(case, scales)


def test_prefill_fp8_mma_query_tiles_of_different_size():
    # a 700-token chunk spans three 256-row query tiles; the middle one is 16x
    # larger, so each tile needs its own scale
    case = synth.make_case("bf16", [700, 40], [100, 300], 8, 2, 0, 1000, seed=197)
    q = case.q.copy()
    q[256:512] *= 16.0
    case.q = q.astype(np.float32)
    _run(case, (1 / 64, 1 / 32))


def test_prefill_fp8_mma_empty_chunks_in_batch():
    case = synth.make_case("bf16", [0, 100, 0, 33], [50, 0, 300, 500], 32, 4, 64, 100, seed=199)
    _run(case, (1 / 64, 1 / 32))


def test_prefill_fp8_mma_repeatable():
    case = synth.make_case("bf16", [300, 90], [0, 700], 32, 4, 0, 2048, seed=198)
    gc = GpuCase(case, fp8_scales=(1 / 64, 1 / 32))
    gc.sconv()
    o1, l1 = gc.prefill_fp8_mma()
    o2, l2 = gc.prefill_fp8_mma()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["full_prefill_32k", "swa_prefill_8k"])
def test_prefill_fp8_mma_full_size_sampled(name):
    # the full-size workloads over an E4M3 cache, 48 rows per sequence (a
    # third of them among the last 256, where the most keys are visible)
    wl = synth.WORKLOADS[name]
    case = synth.workload_case(wl, seed=0)
    rng = np.random.default_rng(7)
    rows = []
    for b in range(len(case.q_lens)):
        n = int(case.q_lens[b])
        r = np.concatenate([rng.choice(n - 256, 32, replace=False), n - 256 + rng.choice(256, 16, replace=False)])
        rows.append(np.sort(r))
    _run(case, (1 / 64, 1 / 64), rows)
