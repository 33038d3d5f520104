"""Benchmark of the Inkling attention-block hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  inkattn_sconv            (K/V short convolution + paged KV-cache write)
  inkattn_relattn_prefill  (relative-position GQA attention over the chunk)
on the full-causal prefill workload (batch 2, T=32768, Hq=32, Hkv=4, d=128,
R=32768, bf16, paged KV block 128), the largest workload that fits one GPU.
value = its attention FLOP per step / step time; roofline = the prefill
kernel alone (HIP events on its launch stream); sconv = the K/V sconv and
cache write alone, in GB/s.

Further legs in the same JSON line:
  prefill_32k_fp8_mma  the headline workload over an E4M3 KV cache with FP8
                 matrix products (Q and P rounded to E4M3), against the FP8
                 MFMA peak
  prefill_8k     the 8K sliding-window prefill step (T=8192, window 2048)
  prefill_fp8    the same over an E4M3 KV cache (pages converted to bf16)
  prefill_8k_fp8_mma  the 8K workload with FP8 matrix products
  decode         16K sliding-window decode (64 sequences, window 4096):
                 one-token sconv + split-K decode (+ merge when split)
  decode_1m      1M-context full-attention decode (4 sequences): split-K
                 pass + LSE merge, timed together; decode_1m_fp8 over E4M3
  decode_mtp     MTP verification: 9 query tokens per sequence, 16K window
  decode_fp8     the 16K decode over an E4M3 cache
  sconv_out      the sconv of a plain [tokens][channels] activation
  ceilings       a dense bf16 MFMA loop (with its shader clock), a 4 GiB
                 streaming read and a 1 GiB device copy, measured in the
                 same job
  cpu_baseline   the fp64 oracle on the host cores: the headline workload on
                 a stratified sample (extrapolated by pair count), the tiny
                 and 8K prefill in full, the 16K and 1M decode on some of
                 their sequences
Decode legs are also timed with a 1 GiB streaming read before every step
(L2 and MALL evicted).  Before the warmup steps of each leg, about
--steady-s seconds of untimed steps bring the shader clock to its sustained
level.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--steady-s S]
                       [--no-cpu-baseline] [--no-prefill-8k] [--no-decode]
                       [--no-1m] [--no-16k] [--no-mtp] [--no-fp8] [--no-sconv-out]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rel-attn prefill TFLOP/s & decode KV GB/s per MI355X (% of roofline)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 (E4M3) MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
HEAD_DIM = 128


def valid_pairs(q_len, seq_len, window):
    """Number of (query, key) pairs inside the causal window for one head."""
    pos = np.arange(seq_len - q_len, seq_len, dtype=np.int64)
    n = pos + 1
    if window > 0:
        n = np.minimum(n, window)
    return int(n.sum())


class DeviceCase:
    """Device tensors of one synth case in the library's layouts."""

    def __init__(self, case, torch, fp8_scales=None):
        import attention_sconv_amd as ink
        from attention_sconv_amd import kvcache
        self.case = c = case
        self.fp8 = fp8_scales
        td = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(td)
        idev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        self.dt = ink.BF16 if c.dtype == "bf16" else ink.FP32
        self.q, self.k_pre, self.v_pre = dev(c.q), dev(c.k_pre), dev(c.v_pre)
        self.conv_w, self.conv_state, self.bias = dev(c.conv_w), dev(c.conv_state), dev(c.bias)
        self.state_slot, self.cu = idev(c.state_slot), idev(c.cu_seqlens)
        self.slot_mapping, self.block_table = idev(c.slot_mapping), idev(c.block_table)
        self.seq_lens = idev(c.seq_lens)
        if c.past_k is not None:
            pk = c.past_k if torch.is_tensor(c.past_k) else dev(c.past_k)
            pv = c.past_v if torch.is_tensor(c.past_v) else dev(c.past_v)
            if fp8_scales:
                # the cached context as E4M3 codes (torch's float8_e4m3fn cast)
                pk, pv = [(x.float() / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
                          .view(torch.uint8) for x, s in ((pk, fp8_scales[0]),
                                                          (pv, fp8_scales[1]))]
            self.k_cache, self.v_cache = kvcache.from_slots(pk, pv)
            del pk, pv
            c.past_k = c.past_v = None
        else:
            self.k_cache, self.v_cache = kvcache.alloc(c.num_blocks, c.num_kv_heads,
                                                       "fp8" if fp8_scales else c.dtype)
            self.k_cache.zero_()
            self.v_cache.zero_()
        self.out = torch.empty_like(self.q)
        self.desc = ink.make_desc(self.dt, c.num_q_heads, c.num_kv_heads, c.window, c.bias_len)
        self.ink = ink

    def sconv(self):
        c = self.case
        if self.fp8:
            self.ink.inkattn_sconv_fp8(self.dt, c.num_kv_heads, HEAD_DIM, len(c.q_lens),
                                       c.num_tokens, int(c.q_lens.max()), self.k_pre,
                                       self.v_pre, self.conv_w, self.conv_state,
                                       self.state_slot, self.cu, self.slot_mapping,
                                       self.fp8[0], self.fp8[1], self.k_cache, self.v_cache)
            return
        self.ink.inkattn_sconv(self.dt, c.num_kv_heads, HEAD_DIM, len(c.q_lens), c.num_tokens,
                               int(c.q_lens.max()), self.k_pre, self.v_pre, self.conv_w,
                               self.conv_state, self.state_slot, self.cu, self.slot_mapping,
                               self.k_cache, self.v_cache)

    def prefill(self):
        c = self.case
        self.ink.inkattn_relattn_prefill(self.desc, len(c.q_lens), c.num_tokens,
                                         int(c.q_lens.max()), self.q, self.k_cache,
                                         self.v_cache, self.block_table,
                                         self.block_table.shape[1], self.cu, self.seq_lens,
                                         self.bias, self.out, None)

    def setup_decode(self, torch):
        c = self.case
        B, L = len(c.q_lens), int(c.seq_lens.max())
        self.num_splits = self.ink.inkattn_relattn_decode_num_splits(self.desc, B, L)
        self.ws_bytes = self.ink.inkattn_relattn_decode_workspace_size(self.desc, B, L, 0)
        self.ws = torch.empty(self.ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")

    def decode(self):
        c = self.case
        self.ink.inkattn_relattn_decode(self.desc, len(c.q_lens), int(c.seq_lens.max()),
                                        self.q, self.k_cache, self.v_cache, self.block_table,
                                        self.block_table.shape[1], self.seq_lens, self.bias,
                                        self.out, None, 0, self.ws, self.ws_bytes)

    def setup_decode_mq(self, torch):
        c = self.case
        B, L, Q = len(c.q_lens), int(c.seq_lens.max()), int(c.q_lens.max())
        self.num_splits = self.ink.inkattn_relattn_decode_mq_num_splits(self.desc, B, Q, L)
        self.ws_bytes = self.ink.inkattn_relattn_decode_mq_workspace_size(
            self.desc, B, c.num_tokens, Q, L, 0)
        self.ws = torch.empty(self.ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")

    def decode_fp8(self):
        c = self.case
        self.ink.inkattn_relattn_decode_fp8(self.desc, len(c.q_lens), c.num_tokens,
                                            int(c.q_lens.max()), int(c.seq_lens.max()), self.q,
                                            self.k_cache, self.v_cache, self.fp8[0],
                                            self.fp8[1], self.block_table,
                                            self.block_table.shape[1], self.cu, self.seq_lens,
                                            self.bias, self.out, None, 0, self.ws,
                                            self.ws_bytes)

    def setup_prefill_fp8(self, torch):
        c = self.case
        self.pf8_ws_bytes = self.ink.inkattn_relattn_prefill_fp8_workspace_size(
            self.desc, len(c.q_lens), self.block_table.shape[1])
        self.pf8_ws = torch.empty(self.pf8_ws_bytes // 4 + 4, dtype=torch.float32,
                                  device="cuda")

    def prefill_fp8(self):
        c = self.case
        self.ink.inkattn_relattn_prefill_fp8(self.desc, len(c.q_lens), c.num_tokens,
                                             int(c.q_lens.max()), self.q, self.k_cache,
                                             self.v_cache, self.fp8[0], self.fp8[1],
                                             self.block_table, self.block_table.shape[1],
                                             self.cu, self.seq_lens, self.bias, self.out, None,
                                             self.pf8_ws, self.pf8_ws_bytes)

    def prefill_fp8_mma(self):
        c = self.case
        self.ink.inkattn_relattn_prefill_fp8_mma(self.desc, len(c.q_lens), c.num_tokens,
                                                 int(c.q_lens.max()), self.q, self.k_cache,
                                                 self.v_cache, self.fp8[0], self.fp8[1],
                                                 self.block_table, self.block_table.shape[1],
                                                 self.cu, self.seq_lens, self.bias, self.out,
                                                 None)

    def decode_mq(self):
        c = self.case
        self.ink.inkattn_relattn_decode_mq(self.desc, len(c.q_lens), c.num_tokens,
                                           int(c.q_lens.max()), int(c.seq_lens.max()), self.q,
                                           self.k_cache, self.v_cache, self.block_table,
                                           self.block_table.shape[1], self.cu, self.seq_lens,
                                           self.bias, self.out, None, 0, self.ws, self.ws_bytes)


def recorded_field(profile, sources, field):
    """Field `field` of profiles/<profile> (a rocprofv3 counter summary), or
    None when the kernel's sources have changed since those counters were
    taken (hash mismatch)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        fields = dict(l.split(":", 1) for l in open(path).read().splitlines() if ":" in l)
    except OSError:
        return None
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    recorded = fields.get("source_sha256_16", "").split()
    if not recorded or recorded[0] != h.hexdigest()[:16] or field not in fields:
        return None
    return float(fields[field].split()[0])


def recorded_traffic(profile, sources):
    """HBM bytes per launch recorded by the rocprofv3 FETCH_SIZE/WRITE_SIZE
    passes summarised in profiles/<profile>, or None when the kernel's
    sources have changed since those counters were taken (hash mismatch)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        fields = dict(l.split(":", 1) for l in open(path).read().splitlines() if ":" in l)
    except OSError:
        return None
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    recorded = fields.get("source_sha256_16", "").split()
    if not recorded or recorded[0] != h.hexdigest()[:16]:
        return None
    return int(fields["traffic_bytes_per_launch"].strip())


def steady_clocks(torch, fn_step, seconds):
    """Run the step back to back for about ``seconds`` before any warmup or
    timed step: the GPU raises its shader clock only under sustained load,
    and a few milliseconds of work straight after setup would otherwise be
    timed at a lower clock than a serving loop runs at.  Returns the number
    of steps run (none of them is timed)."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn_step(None)
        n += 8
        torch.cuda.synchronize()
    return n


def time_region(torch, fn_step, fn_kernel, steps, warmup, between=None):
    """Run warmup untimed steps, then `steps` timed steps.  Returns
    (ms per step, list of per-step ms of the kernel of interest), the latter
    from event pairs recorded around that kernel on the launch stream.  With
    ``between``, it runs before every step (outside the kernel's events; its
    time is part of ms per step)."""
    for _ in range(warmup):
        if between is not None:
            between()
        fn_step(None)
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        if between is not None:
            between()
        fn_step(pairs[i])
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    return ms_step, [a.elapsed_time(b) for a, b in pairs]


def ceilings(torch, ink):
    """Measured ceilings in this job: a dense bf16 MFMA loop (with the shader
    clock it ran at) and a streaming read of 4 GiB of device memory."""
    groups, iters = 1024, 12000
    out = torch.zeros(3 * groups, dtype=torch.float32, device="cuda")
    ink.inkattn_probe_mfma_bf16(groups, iters, out)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    ink.inkattn_probe_mfma_bf16(groups, iters, out)
    e[1].record()
    torch.cuda.synchronize()
    flop = groups * iters * ink.PROBE_MFMA_WAVES * ink.PROBE_MFMA_CHAINS * 32768
    mfma = flop / (e[0].elapsed_time(e[1]) * 1e-3) / 1e12
    r = out.view(groups, 3).cpu().numpy()
    sclk = float(np.median(r[:, 1] / r[:, 2] * 100.0))
    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(7)
    sink = torch.zeros(ink.PROBE_READ_GROUPS, dtype=torch.float32, device="cuda")
    ink.inkattn_probe_stream_read(buf, sink)
    reps = 5
    e[0].record()
    for _ in range(reps):
        ink.inkattn_probe_stream_read(buf, sink)
    e[1].record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9
    # read + write: a device-to-device copy of 1 GiB (the runtime's copy
    # kernel), bytes read plus bytes written per second
    half = buf[: (1 << 30) // 4]
    dst = torch.empty_like(half)
    dst.copy_(half)
    e[0].record()
    for _ in range(reps):
        dst.copy_(half)
    e[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * reps / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9
    del buf, half, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "sclk_mhz_under_mfma": round(sclk),
            "hbm_read_gbs": round(gbs, 1), "hbm_copy_gbs": round(copy_gbs, 1),
            "note": "inkattn_probe_mfma_bf16 (1024 groups x 8 waves x 8 chains of "
                    "32x32x16 bf16), inkattn_probe_stream_read (4 GiB, 256 groups x "
                    "256 threads x 8 loads of 16 B in flight) and a 1 GiB device copy "
                    "(read + write bytes), same job"}


# ---------------------------------------------------------------- CPU baseline
def _cores():
    """Host cores: os.cpu_count(), the affinity set, and the BLAS threads the
    oracle's matrix products run on (its elementwise numpy work is one
    thread)."""
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return nproc, affinity, min(blas, affinity)


def _oracle_prefill_sample(case, wl, blocks_per_seq):
    """The oracle on a workload's prefill step: sconv of every token, then
    attention of whole 256-row blocks of queries (all heads), either every
    block (``blocks_per_seq`` None) or that many blocks per sequence at
    stratified positions.  Returns (seconds, attention FLOP computed,
    estimated seconds of the whole step, rows computed)."""
    import oracle
    c = case
    T, G = wl.q_len, wl.num_q_heads // wl.num_kv_heads
    nb = (T + 255) // 256
    t0 = time.perf_counter()
    k_new, v_new, _ = oracle.sconv_batch(c.k_pre, c.v_pre, c.conv_w, c.conv_state,
                                         c.state_slot, c.cu_seqlens)
    t_sconv = time.perf_counter() - t0
    done_pairs = 0
    rows_done = 0
    t_attn = 0.0
    for b in range(wl.batch):
        if blocks_per_seq is None:
            blocks = range(nb)
        else:
            blocks = sorted(set(int(x) for x in
                                np.linspace(0, nb - 1, blocks_per_seq).round().tolist()))
        s0 = b * T
        K = k_new[s0:s0 + T].reshape(T, wl.num_kv_heads, HEAD_DIM)
        V = v_new[s0:s0 + T].reshape(T, wl.num_kv_heads, HEAD_DIM)
        for blk in blocks:
            rows = np.arange(256 * blk, min(256 * blk + 256, T))
            t1 = time.perf_counter()
            oracle.relattn_prefill(c.q[s0:s0 + T], K, V, c.bias, wl.window, G, rows=rows)
            t_attn += time.perf_counter() - t1
            n = rows + 1 if wl.window == 0 else np.minimum(rows + 1, wl.window)
            done_pairs += int(n.sum())
            rows_done += len(rows)
    total_pairs = valid_pairs(wl.q_len, wl.seq_len, wl.window) * wl.batch
    est = t_sconv + t_attn * total_pairs / done_pairs
    return (t_sconv + t_attn, 4 * HEAD_DIM * done_pairs * wl.num_q_heads, est, rows_done)


def _oracle_decode_sample(case, wl, seqs):
    """The oracle on a decode step for the given sequences: sconv of their new
    token through the state, then attention of the query over the cached
    context gathered through the block table (all heads).  Returns
    (seconds, K+V bytes attended)."""
    import oracle
    c = case
    G = wl.num_q_heads // wl.num_kv_heads
    H = wl.num_kv_heads
    t = 0.0
    nbytes = 0
    for b in seqs:
        L = int(c.seq_lens[b])
        lo = max(0, L - wl.window) if wl.window else 0
        sl = slice(int(c.cu_seqlens[b]), int(c.cu_seqlens[b + 1]))
        st = c.conv_state[int(c.state_slot[b])]
        t0 = time.perf_counter()
        k_new, _ = oracle.sconv_sequence(c.k_pre[sl], c.conv_w[0], st[0])
        v_new, _ = oracle.sconv_sequence(c.v_pre[sl], c.conv_w[1], st[1])
        slots = oracle.slots_for(c.block_table[b], np.arange(lo, L - 1))
        K = np.zeros((L, H, HEAD_DIM))
        V = np.zeros((L, H, HEAD_DIM))
        K[lo:L - 1] = c.past_k[slots]
        V[lo:L - 1] = c.past_v[slots]
        K[L - 1] = k_new.reshape(H, HEAD_DIM)
        V[L - 1] = v_new.reshape(H, HEAD_DIM)
        oracle.relattn_decode(c.q[b], K, V, c.bias, wl.window, G)
        t += time.perf_counter() - t0
        nbytes += (L - lo) * H * HEAD_DIM * 2 * 2
    return t, nbytes


def cpu_baselines(torch, headline_case):
    """The fp64 oracle timed on the host cores (a reported baseline, not a
    target): the headline workload on a stratified sample of whole query
    blocks, extrapolated by pair count; the tiny and 8K prefill workloads in
    full; the 16K decode on 8 of its 64 sequences and the 1M decode on one of
    its four, each extrapolated per sequence."""
    import oracle  # noqa: F401  (the oracle is this leg's whole subject)
    import synth
    nproc, affinity, cores = _cores()
    out = {}
    wl3 = synth.WORKLOADS["full_prefill_32k"]
    t, fl, est, rows = _oracle_prefill_sample(headline_case, wl3, 3)
    total = 4 * HEAD_DIM * valid_pairs(wl3.q_len, wl3.seq_len, wl3.window) \
        * wl3.num_q_heads * wl3.batch
    out["headline"] = {
        "value": round(total / est / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
        "nproc": nproc, "affinity": affinity, "kind": "oracle",
        "sample": f"{wl3.name}: sconv of all {wl3.batch * wl3.q_len} tokens + attention of "
                  f"{rows} query rows (3 stratified 256-row blocks per sequence, all "
                  f"{wl3.num_q_heads} heads) in {t:.1f} s; extrapolated by valid pairs to "
                  f"{est:.0f} s for the whole step; fp64 numpy"}
    for name in ("tiny_fp32_swa_prefill", "swa_prefill_8k"):
        wl = synth.WORKLOADS[name]
        case = synth.workload_case(wl, seed=0)
        t, fl, est, rows = _oracle_prefill_sample(case, wl, None)
        out[name] = {"value": round(fl / t / 1e12, 5), "unit": "TFLOP/s", "seconds": round(t, 2),
                     "cores": cores, "mode": "full", "kind": "oracle",
                     "sample": f"one whole step: sconv + all {rows} rows x {wl.num_q_heads} heads"}
        del case
    for name, nseq in (("swa_decode_16k", 8), ("full_decode_1m", 1)):
        wl = synth.WORKLOADS[name]
        case = synth.make_case(wl.dtype, [1] * nseq, [wl.seq_len - 1] * nseq, wl.num_q_heads,
                               wl.num_kv_heads, wl.window, wl.bias_len, seed=0)
        t, nbytes = _oracle_decode_sample(case, wl, range(nseq))
        out[name] = {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "seconds": round(t, 2),
                     "cores": cores, "mode": "extrapolated", "kind": "oracle",
                     "est_seconds_full_batch": round(t * wl.batch / nseq, 1),
                     "sample": f"{nseq} of {wl.batch} sequences: sconv of the new token + "
                               f"attention over {min(wl.window or wl.seq_len, wl.seq_len)} "
                               f"keys, all {wl.num_q_heads} heads"}
        del case
    head = out.pop("headline")
    head["other_workloads"] = out
    return head


# ---------------------------------------------------------------- legs
def sconv_bytes(c, elem_bytes, cache_elem_bytes=None):
    """Algorithmic bytes of one K/V sconv call: the pre-conv rows read, the
    cache rows written, each sequence's 3-row state read and written, and
    the taps."""
    cb = elem_bytes if cache_elem_bytes is None else cache_elem_bytes
    C = c.num_kv_heads * HEAD_DIM
    n, b = c.num_tokens, len(c.q_lens)
    return 2 * n * C * elem_bytes + 2 * n * C * cb + 2 * (2 * 3 * C * elem_bytes) * b \
        + 2 * C * 4 * elem_bytes


def time_sconv(torch, dc, steps, warmup):
    """The K/V sconv + cache write alone (HIP events on its stream)."""
    def st(ev):
        if ev is not None:
            ev[0].record()
        dc.sconv()
        if ev is not None:
            ev[1].record()
    steady_clocks(torch, st, 0.05)
    _, ks = time_region(torch, st, None, steps, warmup)
    ms = float(np.median(ks))
    nbytes = sconv_bytes(dc.case, 2 if dc.case.dtype == "bf16" else 4, 1 if dc.fp8 else None)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"tokens": dc.case.num_tokens, "sequences": len(dc.case.q_lens),
            "ms_median": round(ms, 5), "ms_min": round(min(ks), 5), "bytes": nbytes,
            "achieved": round(gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def prefill_leg(torch, args, name, result_key=None, with_sconv_leg=True):
    """sconv + prefill steps of a prefill workload.  Returns (summary dict,
    device case)."""
    import synth
    wl = synth.WORKLOADS[name]
    case = synth.workload_case(wl, seed=0)
    dc = DeviceCase(case, torch)
    pairs = valid_pairs(wl.q_len, wl.seq_len, wl.window) * wl.num_q_heads * wl.batch
    flop = 4 * HEAD_DIM * pairs

    def step(ev):
        dc.sconv()
        if ev is not None:
            ev[0].record()
        dc.prefill()
        if ev is not None:
            ev[1].record()

    print(f"[bench] prefill {wl.name}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    n_steady = steady_clocks(torch, step, args.steady_s)
    ms_step, ks = time_region(torch, step, None, args.steps, args.warmup)
    ms = sum(ks) / len(ks)
    tf = flop / (ms * 1e-3) / 1e12
    prof = f"prefill_bf16_{wl.name}"
    srcs = ["attention_sconv_amd/csrc/prefill.hip", "attention_sconv_amd/csrc/device_common.h"]
    summary = {
        "workload": wl.name + ": " + wl.description + ", paged KV block 128",
        "ms_per_step": round(ms_step, 4),
        "step_tflops": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(prof + ".traffic.txt", srcs),
                     "mfma_busy_pct": recorded_field(prof + ".mfma.txt", srcs, "mfma_busy_pct"),
                     "kernel": "prefill_kernel<bf16>", "ms": round(ms, 4),
                     "ms_median": round(float(np.median(ks)), 4), "ms_min": round(min(ks), 4),
                     "algorithmic_flop": flop},
        "steady_clock_steps": n_steady,
    }
    if with_sconv_leg:
        print(f"[bench] sconv cache write, {wl.name} chunk", file=sys.stderr, flush=True)
        summary["sconv"] = time_sconv(torch, dc, max(args.steps, 20), args.warmup)
        summary["sconv"]["traffic"] = recorded_traffic(
            f"sconv_write_bf16_{wl.name}.traffic.txt",
            ["attention_sconv_amd/csrc/sconv.hip", "attention_sconv_amd/csrc/device_common.h"])
    return summary, dc, flop


def prefill_fp8_mma_leg(torch, args, name, bf16_ms=None):
    """sconv (E4M3 cache write, scales 1/64) + the prefill with FP8 matrix
    products on a prefill workload.  The roofline is the FP8 (E4M3) MFMA
    peak; ``time_vs_bf16`` compares with the bf16 prefill of the same
    workload measured earlier in this run."""
    import synth
    wl = synth.WORKLOADS[name]
    dc = DeviceCase(synth.workload_case(wl, seed=0), torch, fp8_scales=(1 / 64, 1 / 64))
    flop = 4 * HEAD_DIM * valid_pairs(wl.q_len, wl.seq_len, wl.window) * wl.num_q_heads * wl.batch

    def step(ev):
        dc.sconv()
        if ev is not None:
            ev[0].record()
        dc.prefill_fp8_mma()
        if ev is not None:
            ev[1].record()

    print(f"[bench] prefill {wl.name}, E4M3 cache, FP8 products", file=sys.stderr, flush=True)
    steady_clocks(torch, step, args.steady_s)
    ms_step, ks = time_region(torch, step, None, args.steps, args.warmup)
    ms = sum(ks) / len(ks)
    tf = flop / (ms * 1e-3) / 1e12
    srcs = ["attention_sconv_amd/csrc/prefill_f8.hip", "attention_sconv_amd/csrc/prefill_common.h",
            "attention_sconv_amd/csrc/device_common.h"]
    out = {
        "workload": wl.name + " with an E4M3 KV cache (scales 1/64), Q and P rounded to E4M3",
        "ms_per_step": round(ms_step, 4),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(f"prefill_f8_{wl.name}.traffic.txt", srcs),
                     "kernel": "prefill_f8_kernel", "ms": round(ms, 4),
                     "ms_median": round(float(np.median(ks)), 4), "ms_min": round(min(ks), 4),
                     "algorithmic_flop": flop},
        "note": "inkattn_relattn_prefill_fp8_mma: v_mfma_f32_32x32x64_f8f6f4 for Q K^T and P V",
    }
    if bf16_ms:
        out["time_vs_bf16"] = round(ms / bf16_ms, 3)
    del dc
    torch.cuda.empty_cache()
    return out


def decode_leg(torch, args, name, fp8=False, flush=True):
    """sconv (one token per sequence) + split-K decode + merge steps of a
    decode workload, bf16 cache or E4M3 cache (scales 1/64)."""
    import synth
    import attention_sconv_amd as ink
    wl = synth.WORKLOADS[name]
    case = synth.workload_case(wl, seed=0, past_device="cuda")
    dd = DeviceCase(case, torch, fp8_scales=(1 / 64, 1 / 64) if fp8 else None)
    if fp8:
        dd.setup_decode_mq(torch)
        fn = dd.decode_fp8
    else:
        dd.setup_decode(torch)
        fn = dd.decode
    keys = min(wl.window, wl.seq_len) if wl.window else wl.seq_len
    kv_bytes = wl.batch * wl.num_kv_heads * 2 * keys * HEAD_DIM * (1 if fp8 else 2)

    def dstep(ev):
        dd.sconv()
        if ev is not None:
            ev[0].record()
        fn()
        if ev is not None:
            ev[1].record()

    print(f"[bench] decode {wl.name}{' with an FP8 cache' if fp8 else ''}", file=sys.stderr,
          flush=True)
    d_steps = max(args.steps, 20)
    steady_clocks(torch, dstep, args.steady_s)
    ms_step, ks = time_region(torch, dstep, None, d_steps, args.warmup)
    ms = sum(ks) / len(ks)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    res = {"workload": wl.name + ": " + wl.description
           + (" with an E4M3 KV cache (scales 1/64)" if fp8 else ""),
           "ms_per_step": round(ms_step, 4), "ms_decode": round(ms, 4),
           "ms_decode_median": round(float(np.median(ks)), 4),
           "ms_decode_min": round(min(ks), 4), "num_splits": dd.num_splits,
           "kv_bytes": kv_bytes, "achieved": round(gbs, 1), "unit": "GB/s",
           "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4)}
    if flush:
        # the same with a streaming read of 1 GiB before every step, which
        # evicts the attended K/V from L2 and the 256 MB MALL (clean lines,
        # so no write-back competes with the decode)
        fl = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.zeros(ink.PROBE_READ_GROUPS, dtype=torch.float32, device="cuda")
        _, fks = time_region(torch, dstep, None, d_steps, args.warmup,
                             between=lambda: ink.inkattn_probe_stream_read(fl, sink))
        del fl
        f_ms = float(np.median(fks))
        f_gbs = kv_bytes / (f_ms * 1e-3) / 1e9
        res["flushed"] = {"ms_median": round(f_ms, 4), "ms_min": round(min(fks), 4),
                          "achieved": round(f_gbs, 1), "frac": round(f_gbs / PEAK_HBM_GBS, 4),
                          "note": "1 GiB streaming read before every step (L2 and MALL "
                                  "evicted)"}
    return res, dd, ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip every decode leg")
    ap.add_argument("--no-prefill-8k", action="store_true",
                    help="skip the 8K sliding-window prefill leg")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-context decode legs")
    ap.add_argument("--no-16k", action="store_true",
                    help="skip the 16K sliding-window decode legs (bf16 and E4M3 cache)")
    ap.add_argument("--no-mtp", action="store_true",
                    help="skip the MTP-verification decode leg")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the legs with an FP8 (E4M3) KV cache")
    ap.add_argument("--no-sconv-out", action="store_true",
                    help="skip the leg that times the sconv of a plain activation tensor")
    ap.add_argument("--steady-s", type=float, default=0.3,
                    help="seconds of untimed back-to-back steps before the warmup steps, "
                         "so that the timed steps run at the sustained shader clock")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the bench, run one plain device-to-device copy of this "
                         "many bytes (reference kernel for HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU split is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_sconv_amd as ink

    # ---------------- headline: sconv + prefill on the 32K full-causal workload
    head, dc, flop = prefill_leg(torch, args, "full_prefill_32k")
    headline_case = dc.case
    ms_step = head["ms_per_step"]
    result = {
        "metric": METRIC,
        "value": head["step_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"] + ", step = sconv + prefill",
                   "global_batch": 2, "seq_len": 32768, "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "sconv": head["sconv"],
        "steady_clock_steps": head["steady_clock_steps"],
    }
    del dc
    torch.cuda.empty_cache()
    if not args.no_fp8:
        result["prefill_32k_fp8_mma"] = prefill_fp8_mma_leg(torch, args, "full_prefill_32k",
                                                            head["roofline"]["ms"])

    # ---------------- the 8K sliding-window prefill (sconv + prefill)
    if not args.no_prefill_8k:
        p8, dc8, flop8 = prefill_leg(torch, args, "swa_prefill_8k")
        result["config"]["prefill_8k"] = p8["workload"]
        result["prefill_8k"] = p8
        del dc8
        if not args.no_fp8:
            import synth
            wl = synth.WORKLOADS["swa_prefill_8k"]
            fpd = DeviceCase(synth.workload_case(wl, seed=0), torch, fp8_scales=(1 / 64, 1 / 64))
            fpd.setup_prefill_fp8(torch)

            def fpstep(ev):
                fpd.sconv()
                if ev is not None:
                    ev[0].record()
                fpd.prefill_fp8()
                if ev is not None:
                    ev[1].record()

            print("[bench] prefill swa_prefill_8k with an FP8 cache", file=sys.stderr,
                  flush=True)
            steady_clocks(torch, fpstep, args.steady_s)
            _, fks = time_region(torch, fpstep, None, args.steps, args.warmup)
            f_ms = sum(fks) / len(fks)
            p8_ms = p8["roofline"]["ms"]
            result["prefill_fp8"] = {
                "workload": wl.name + " with an E4M3 KV cache (scales 1/64)",
                "ms": round(f_ms, 4), "ms_median": round(float(np.median(fks)), 4),
                "achieved": round(flop8 / (f_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "frac": round(flop8 / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "time_vs_bf16_cache": round(f_ms / p8_ms, 3),
                "note": "inkattn_relattn_prefill_fp8: page conversion to a bf16 workspace + "
                        "prefill kernel, both inside the timed call"}
            del fpd
            result["prefill_8k_fp8_mma"] = prefill_fp8_mma_leg(torch, args, "swa_prefill_8k",
                                                               p8["roofline"]["ms"])
        torch.cuda.empty_cache()

    # ---------------- decode: 16K sliding window (64 sequences)
    if not args.no_decode and not args.no_16k:
        res, dd, d_ms = decode_leg(torch, args, "swa_decode_16k")
        res["traffic"] = recorded_traffic("decode_split_bf16_swa_decode_16k.traffic.txt",
                                          ["attention_sconv_amd/csrc/decode.hip",
                                           "attention_sconv_amd/csrc/device_common.h"])
        print("[bench] sconv cache write, one token per sequence", file=sys.stderr, flush=True)
        res["sconv"] = time_sconv(torch, dd, max(args.steps, 20), args.warmup)
        result["decode"] = res
        del dd
        torch.cuda.empty_cache()

    # ---------------- decode: 1M full attention (4 sequences, split-K + merge)
    if not args.no_decode and not args.no_1m:
        res, dd, m1_ms = decode_leg(torch, args, "full_decode_1m")
        res["traffic"] = recorded_traffic("decode_split_bf16_full_decode_1m.traffic.txt",
                                          ["attention_sconv_amd/csrc/decode.hip",
                                           "attention_sconv_amd/csrc/device_common.h"])
        res["merge_traffic"] = recorded_traffic("decode_merge_bf16_full_decode_1m.traffic.txt",
                                                ["attention_sconv_amd/csrc/decode.hip",
                                                 "attention_sconv_amd/csrc/device_common.h"])
        res["note"] = ("split pass + LSE merge timed together (HIP events around the call); "
                       "traffic: the split kernel, merge_traffic: the merge kernel")
        result["decode_1m"] = res
        del dd
        torch.cuda.empty_cache()
        if not args.no_fp8:
            res8, dd, m8_ms = decode_leg(torch, args, "full_decode_1m", fp8=True)
            res8["speedup_vs_bf16_cache"] = round(m1_ms / m8_ms, 3)
            res8["traffic"] = recorded_traffic("decode_split_fp8_full_decode_1m.traffic.txt",
                                               ["attention_sconv_amd/csrc/decode.hip",
                                                "attention_sconv_amd/csrc/device_common.h"])
            result["decode_1m_fp8"] = res8
            del dd
            torch.cuda.empty_cache()

    # ---------------- MTP verification: 9 query tokens per sequence
    if not args.no_decode and not args.no_mtp:
        import synth
        mwl = synth.WORKLOADS["swa_decode_16k_mtp9"]
        md = DeviceCase(synth.workload_case(mwl, seed=0, past_device="cuda"), torch)
        md.setup_decode_mq(torch)
        m_keys = min(mwl.window + mwl.q_len - 1, mwl.seq_len)
        m_kv_bytes = mwl.batch * mwl.num_kv_heads * 2 * m_keys * HEAD_DIM * 2
        m_pairs = valid_pairs(mwl.q_len, mwl.seq_len, mwl.window) * mwl.batch * mwl.num_q_heads

        def mstep(ev):
            md.sconv()
            if ev is not None:
                ev[0].record()
            md.decode_mq()
            if ev is not None:
                ev[1].record()

        print(f"[bench] decode {mwl.name}", file=sys.stderr, flush=True)
        d_steps = max(args.steps, 20)
        steady_clocks(torch, mstep, args.steady_s)
        _, mks = time_region(torch, mstep, None, d_steps, args.warmup)
        m_ms = sum(mks) / len(mks)
        m_gbs = m_kv_bytes / (m_ms * 1e-3) / 1e9
        result["decode_mtp"] = {
            "workload": mwl.name + ": " + mwl.description,
            "ms_decode": round(m_ms, 4), "ms_decode_median": round(float(np.median(mks)), 4),
            "num_splits": md.num_splits, "kv_bytes": m_kv_bytes,
            "achieved": round(m_gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(m_gbs / PEAK_HBM_GBS, 4),
            "tflops": round(4 * HEAD_DIM * m_pairs / (m_ms * 1e-3) / 1e12, 2),
            "traffic": recorded_traffic(
                "decode_mqr_bf16_swa_decode_16k_mtp9.traffic.txt",
                ["attention_sconv_amd/csrc/decode_mqr.hip",
                 "attention_sconv_amd/csrc/device_common.h"]),
            "note": "inkattn_relattn_decode_mq; the 72 (token, head) columns of a kv-head "
                    "group share one read of its K/V: each of 4 waves holds every column "
                    "and a quarter of the keys, loaded straight into its registers",
        }
        if "decode" in result:
            result["decode_mtp"]["time_vs_one_token_decode"] = round(
                m_ms / result["decode"]["ms_decode"], 3)
        del md
        torch.cuda.empty_cache()
        if not args.no_fp8:
            mf = DeviceCase(synth.workload_case(mwl, seed=0, past_device="cuda"), torch,
                            fp8_scales=(1 / 64, 1 / 64))
            mf.setup_decode_mq(torch)

            def mfstep(ev):
                mf.sconv()
                if ev is not None:
                    ev[0].record()
                mf.decode_fp8()
                if ev is not None:
                    ev[1].record()

            print(f"[bench] decode {mwl.name} with an FP8 cache", file=sys.stderr, flush=True)
            steady_clocks(torch, mfstep, args.steady_s)
            _, mfks = time_region(torch, mfstep, None, d_steps, args.warmup)
            mf_ms = sum(mfks) / len(mfks)
            mf_gbs = m_kv_bytes / 2 / (mf_ms * 1e-3) / 1e9
            result["decode_mtp"]["fp8_cache"] = {
                "ms_decode": round(mf_ms, 4),
                "ms_decode_median": round(float(np.median(mfks)), 4),
                "kv_bytes": m_kv_bytes // 2, "achieved": round(mf_gbs, 1), "unit": "GB/s",
                "frac": round(mf_gbs / PEAK_HBM_GBS, 4),
                "speedup_vs_bf16_cache": round(m_ms / mf_ms, 3),
                "traffic": recorded_traffic(
                    "decode_mqr_fp8_swa_decode_16k_mtp9.traffic.txt",
                    ["attention_sconv_amd/csrc/decode_mqr.hip",
                     "attention_sconv_amd/csrc/device_common.h"]),
                "note": "inkattn_relattn_decode_fp8 on the same workload (E4M3 codes, "
                        "scales 1/64)"}
            del mf
            torch.cuda.empty_cache()

    # ---------------- E4M3 cache: the 16K sliding-window decode again
    if not args.no_decode and not args.no_fp8 and not args.no_16k:
        res, dd, f8_ms = decode_leg(torch, args, "swa_decode_16k", fp8=True, flush=False)
        if "decode" in result:
            res["speedup_vs_bf16_cache"] = round(result["decode"]["ms_decode"] / f8_ms, 3)
        res["traffic"] = recorded_traffic("decode_split_fp8_swa_decode_16k.traffic.txt",
                                          ["attention_sconv_amd/csrc/decode.hip",
                                           "attention_sconv_amd/csrc/device_common.h"])
        res["note"] = ("inkattn_sconv_fp8 + inkattn_relattn_decode_fp8; bytes = the E4M3 K+V "
                       "in the attended range")
        result["decode_fp8"] = res
        del dd
        torch.cuda.empty_cache()

    # ---------------- sconv of a plain activation (attention / MoE output)
    if not args.no_sconv_out:
        import synth
        sc = synth.make_sconv_out_case("bf16", [8192] * 4, 4096, seed=0, extra_slots=0)
        td = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(
            torch.bfloat16)
        sx, sw, sst = td(sc.x), td(sc.conv_w), td(sc.conv_state)
        sslot = torch.from_numpy(sc.state_slot).cuda()
        scu = torch.from_numpy(sc.cu_seqlens.astype(np.int32)).cuda()
        sy = torch.empty_like(sx)
        s_bytes = 2 * sx.numel() * 2 + 2 * sst.numel() * 2 + sw.numel() * 2

        def sstep(ev):
            if ev is not None:
                ev[0].record()
            ink.inkattn_sconv_out(ink.BF16, 4096, 4, sx.shape[0], 8192, sx, sw, sst, sslot,
                                  scu, sy)
            if ev is not None:
                ev[1].record()

        print("[bench] sconv_out", file=sys.stderr, flush=True)
        steady_clocks(torch, sstep, 0.1)
        _, sks = time_region(torch, sstep, None, max(args.steps, 20), args.warmup)
        s_ms = float(np.median(sks))
        s_gbs = s_bytes / (s_ms * 1e-3) / 1e9
        result["sconv_out"] = {
            "workload": "4 x 8192 tokens x 4096 channels, bf16 (a stand-in width)",
            "ms_median": round(s_ms, 4), "ms_min": round(min(sks), 4), "bytes": s_bytes,
            "achieved": round(s_gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(s_gbs / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(
                "sconv_out_bf16_4x8192x4096.traffic.txt",
                ["attention_sconv_amd/csrc/sconv.hip",
                 "attention_sconv_amd/csrc/device_common.h"]),
            "note": "inkattn_sconv_out; bytes = x read + y written + state read and written "
                    "+ taps",
        }
        del sx, sy, sst

    print("[bench] measured ceilings", file=sys.stderr, flush=True)
    ceil = ceilings(torch, ink)
    result["ceilings"] = ceil
    result["roofline"]["frac_of_measured"] = round(
        result["roofline"]["achieved"] / ceil["mfma_bf16_tflops"], 4)
    # read-only legs against the streaming-read ceiling, the sconv legs (as
    # many bytes written as read) against the copy ceiling
    for key in ("decode", "decode_1m", "decode_1m_fp8", "decode_fp8", "decode_mtp"):
        if key in result:
            result[key]["frac_of_measured"] = round(result[key]["achieved"]
                                                    / ceil["hbm_read_gbs"], 4)
    for leg in (result.get("sconv"), result.get("prefill_8k", {}).get("sconv"),
                result.get("decode", {}).get("sconv"), result.get("sconv_out")):
        if leg:
            leg["frac_of_copy"] = round(leg["achieved"] / ceil["hbm_copy_gbs"], 4)

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baselines(torch, headline_case)

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_bytes"] = n * 4

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
