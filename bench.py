"""Benchmark of the Inkling attention-block hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  inkattn_sconv            (K/V short convolution + paged KV-cache write)
  inkattn_relattn_prefill  (relative-position GQA attention over the chunk)
on the sliding-window prefill workload (batch 1, T=8192, Hq=32, Hkv=4,
d=128, window 2048, R=2048, bf16, paged KV block 128).  The decode half of
the metric (split-K decode + LSE merge, after the one-token sconv) is measured
in the same run on the 16K sliding-window decode workload (batch 64,
L=16384, window 4096) and reported under "decode".

The 32K full-causal prefill workload (batch 2, T=32768, Hq=32, Hkv=4, R=32768)
is timed too, kernel alone, and reported under "prefill_32k"; so are the
MTP9 verification step ("decode_mtp"), the 8K prefill and the 16K decode over
an E4M3 cache ("prefill_fp8", "decode_fp8") and the sconv of a plain activation
("sconv_out").

Prints ONE JSON line.  value = algorithmic attention FLOP per step / step
time; roofline = the prefill kernel alone (HIP events on the launch stream).
cpu_baseline = the fp64 oracle on a bounded sample of the same workload.
ceilings = a dense bf16 MFMA loop (with the shader clock it ran at) and a
4 GiB streaming read, measured in the same job; frac_of_measured divides by
them.  Before the warmup steps of each leg, about --steady-s seconds of
untimed steps bring the shader clock to its sustained level.  Decode is also
timed with a 1 GiB streaming read before every step (L2 and MALL evicted).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--steady-s S]
                       [--no-cpu-baseline] [--no-prefill-32k] [--no-decode]
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
    del buf
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "sclk_mhz_under_mfma": round(sclk),
            "hbm_read_gbs": round(gbs, 1),
            "note": "inkattn_probe_mfma_bf16 (1024 groups x 8 waves x 8 chains of "
                    "32x32x16 bf16) and inkattn_probe_stream_read (4 GiB, 256 groups x "
                    "256 threads x 8 loads of 16 B in flight), same job"}


def cpu_baseline(case, budget_s=10.0):
    """The fp64 oracle on the prefill workload, timed on the host cores: the
    sconv of the chunk, then attention of all query rows (all heads) in
    blocks of 256, repeated until at least ``budget_s`` seconds of work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = 1
    c = case
    G = c.num_q_heads // c.num_kv_heads
    T = int(c.q_lens[0])
    flops = 0
    rows_done = 0
    passes = 0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < budget_s and passes < 8:
        k_new, v_new, _ = oracle.sconv_batch(c.k_pre, c.v_pre, c.conv_w, c.conv_state,
                                             c.state_slot, c.cu_seqlens)
        K = k_new.reshape(T, c.num_kv_heads, HEAD_DIM)
        V = v_new.reshape(T, c.num_kv_heads, HEAD_DIM)
        for s in range(0, T, 256):
            rows = np.arange(s, min(s + 256, T))
            oracle.relattn_prefill(c.q, K, V, c.bias, c.window, G, rows=rows)
            n = rows + 1 if c.window == 0 else np.minimum(rows + 1, c.window)
            flops += int(n.sum()) * 4 * HEAD_DIM * c.num_q_heads
            rows_done += len(rows)
        passes += 1
    dt = time.perf_counter() - t_start
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{passes} full pass(es) of the workload (sconv of {T} tokens + "
                      f"attention of all {T} rows x {c.num_q_heads} heads) in {dt:.1f} s, "
                      f"fp64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill-32k", action="store_true",
                    help="skip the 32K full-causal prefill leg")
    ap.add_argument("--no-mtp", action="store_true",
                    help="skip the MTP-verification decode leg (it launches the decode kernel "
                         "with another shape)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the decode leg with an FP8 (E4M3) KV cache")
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
    import synth

    # ---------------- prefill: sconv + prefill on the 8K SWA workload
    wl = synth.WORKLOADS["swa_prefill_8k"]
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
    ms_prefill = sum(ks) / len(ks)
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (ms_prefill * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + ": " + wl.description + ", paged KV block 128, "
                   "step = sconv + prefill", "global_batch": wl.batch,
                   "seq_len": wl.seq_len, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(
                         "prefill_bf16_swa_prefill_8k.traffic.txt",
                         ["attention_sconv_amd/csrc/prefill.hip",
                          "attention_sconv_amd/csrc/device_common.h"]),
                     "mfma_busy_pct": recorded_field(
                         "prefill_bf16_swa_prefill_8k.mfma.txt",
                         ["attention_sconv_amd/csrc/prefill.hip",
                          "attention_sconv_amd/csrc/device_common.h"], "mfma_busy_pct"),
                     "kernel": "prefill_kernel<bf16>", "ms": round(ms_prefill, 4),
                     "ms_median": round(float(np.median(ks)), 4),
                     "ms_min": round(min(ks), 4),
                     "algorithmic_flop": flop},
        "steady_clock_steps": n_steady,
    }

    # ---------------- the 8K SWA prefill step over an E4M3 cache
    if not args.no_fp8:
        fcase8 = synth.workload_case(wl, seed=0)
        fpd = DeviceCase(fcase8, torch, fp8_scales=(1 / 64, 1 / 64))
        fpd.setup_prefill_fp8(torch)

        def fpstep(ev):
            fpd.sconv()
            if ev is not None:
                ev[0].record()
            fpd.prefill_fp8()
            if ev is not None:
                ev[1].record()

        print(f"[bench] prefill {wl.name} with an FP8 cache", file=sys.stderr, flush=True)
        steady_clocks(torch, fpstep, args.steady_s)
        _, fks = time_region(torch, fpstep, None, args.steps, args.warmup)
        f_ms = sum(fks) / len(fks)
        result["prefill_fp8"] = {
            "workload": wl.name + " with an E4M3 KV cache (scales 1/64)",
            "ms": round(f_ms, 4), "ms_median": round(float(np.median(fks)), 4),
            "achieved": round(flop / (f_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "frac": round(flop / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "time_vs_bf16_cache": round(f_ms / ms_prefill, 3),
            "note": "inkattn_relattn_prefill_fp8: page conversion to a bf16 workspace + "
                    "prefill kernel, both inside the timed call",
        }
        del fpd, fcase8

    # ---------------- prefill on the 32K full-causal workload (kernel alone)
    if not args.no_prefill_32k:
        del dc
        torch.cuda.empty_cache()
        lwl = synth.WORKLOADS["full_prefill_32k"]
        print(f"[bench] prefill {lwl.name}", file=sys.stderr, flush=True)
        lcase = synth.workload_case(lwl, seed=0)
        dc = DeviceCase(lcase, torch)
        dc.sconv()
        l_flop = 4 * HEAD_DIM * valid_pairs(lwl.q_len, lwl.seq_len, lwl.window) \
            * lwl.num_q_heads * lwl.batch

        def lstep(ev):
            if ev is not None:
                ev[0].record()
            dc.prefill()
            if ev is not None:
                ev[1].record()

        steady_clocks(torch, lstep, args.steady_s)
        _, lks = time_region(torch, lstep, None, 5, 2)
        l_ms = sum(lks) / len(lks)
        l_tf = l_flop / (l_ms * 1e-3) / 1e12
        result["prefill_32k"] = {
            "workload": lwl.name + ": " + lwl.description + ", paged KV block 128",
            "kernel": "prefill_kernel<bf16>", "ms": round(l_ms, 3),
            "ms_median": round(float(np.median(lks)), 3), "algorithmic_flop": l_flop,
            "achieved": round(l_tf, 1), "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
            "frac": round(l_tf / PEAK_BF16_TFLOPS, 4),
            "note": "prefill kernel alone (HIP events), 5 timed launches after 2 warmup",
        }
        del lcase

    # ---------------- decode: sconv (1 token/seq) + split-K decode, 16K SWA
    if not args.no_decode:
        del dc
        torch.cuda.empty_cache()
        dwl = synth.WORKLOADS["swa_decode_16k"]
        dcase = synth.workload_case(dwl, seed=0, past_device="cuda")
        dd = DeviceCase(dcase, torch)
        dd.setup_decode(torch)
        kv_bytes = dwl.batch * dwl.num_kv_heads * 2 * min(dwl.window, dwl.seq_len) * HEAD_DIM * 2

        def dstep(ev):
            dd.sconv()
            if ev is not None:
                ev[0].record()
            dd.decode()
            if ev is not None:
                ev[1].record()

        print(f"[bench] decode {dwl.name}", file=sys.stderr, flush=True)
        d_steps = max(args.steps, 20)
        steady_clocks(torch, dstep, args.steady_s)
        d_ms_step, dks = time_region(torch, dstep, None, d_steps, args.warmup)
        d_ms = sum(dks) / len(dks)
        gbs = kv_bytes / (d_ms * 1e-3) / 1e9
        # The same with a streaming read of 1 GiB before every step, which
        # evicts the attended K/V from L2 and the 256 MB MALL (with clean
        # lines, so no write-back competes with the decode): decode then
        # reads HBM.
        import attention_sconv_amd as ink
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.zeros(ink.PROBE_READ_GROUPS, dtype=torch.float32, device="cuda")
        _, fks = time_region(torch, dstep, None, d_steps, args.warmup,
                             between=lambda: ink.inkattn_probe_stream_read(flush, sink))
        del flush
        f_ms = float(np.median(fks))
        f_gbs = kv_bytes / (f_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": dwl.name + ": " + dwl.description,
            "ms_per_step": round(d_ms_step, 4), "ms_decode": round(d_ms, 4),
            "num_splits": dd.num_splits,
            "kv_bytes": kv_bytes, "achieved": round(gbs, 1), "unit": "GB/s",
            "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "ms_decode_median": round(float(np.median(dks)), 4), "ms_decode_min": round(min(dks), 4),
            "flushed": {"ms_median": round(f_ms, 4), "ms_min": round(min(fks), 4),
                        "achieved": round(f_gbs, 1), "frac": round(f_gbs / PEAK_HBM_GBS, 4),
                        "note": "1 GiB streaming read before every step (L2 and MALL evicted)"},
            "traffic": recorded_traffic(
                "decode_split_bf16_swa_decode_16k.traffic.txt",
                ["attention_sconv_amd/csrc/decode.hip",
                 "attention_sconv_amd/csrc/device_common.h"]),
            "note": "achieved/frac: back-to-back steps; flushed: L2/MALL evicted before each step",
        }
        del dd
        torch.cuda.empty_cache()

    # ---------------- MTP verification: 9 query tokens per sequence
    if not args.no_decode and not args.no_mtp:
        mwl = synth.WORKLOADS["swa_decode_16k_mtp9"]
        mcase = synth.workload_case(mwl, seed=0, past_device="cuda")
        md = DeviceCase(mcase, torch)
        md.setup_decode_mq(torch)
        m_keys = min(mwl.window + mwl.q_len - 1, mwl.seq_len)
        m_kv_bytes = mwl.batch * mwl.num_kv_heads * 2 * m_keys * HEAD_DIM * 2
        m_pairs = sum(valid_pairs(mwl.q_len, mwl.seq_len, mwl.window)
                      for _ in range(mwl.batch)) * mwl.num_q_heads

        def mstep(ev):
            md.sconv()
            if ev is not None:
                ev[0].record()
            md.decode_mq()
            if ev is not None:
                ev[1].record()

        print(f"[bench] decode {mwl.name}", file=sys.stderr, flush=True)
        steady_clocks(torch, mstep, args.steady_s)
        m_ms_step, mks = time_region(torch, mstep, None, d_steps, args.warmup)
        m_ms = sum(mks) / len(mks)
        m_gbs = m_kv_bytes / (m_ms * 1e-3) / 1e9
        result["decode_mtp"] = {
            "workload": mwl.name + ": " + mwl.description,
            "ms_decode": round(m_ms, 4), "ms_decode_median": round(float(np.median(mks)), 4),
            "num_splits": md.num_splits, "kv_bytes": m_kv_bytes,
            "achieved": round(m_gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(m_gbs / PEAK_HBM_GBS, 4),
            "tflops": round(4 * HEAD_DIM * m_pairs / (m_ms * 1e-3) / 1e12, 2),
            "time_vs_one_token_decode": round(m_ms / d_ms, 3),
            "traffic": recorded_traffic(
                "decode_mq_bf16_swa_decode_16k_mtp9.traffic.txt",
                ["attention_sconv_amd/csrc/decode_mq.hip",
                 "attention_sconv_amd/csrc/device_common.h"]),
            "note": "inkattn_relattn_decode_mq; the 72 (token, head) columns of a kv-head "
                    "group share one read of its K/V, staged through LDS",
        }
        del md
        torch.cuda.empty_cache()
        if not args.no_fp8:
            # the same verification step over an E4M3 cache
            mcase8 = synth.workload_case(mwl, seed=0, past_device="cuda")
            mf = DeviceCase(mcase8, torch, fp8_scales=(1 / 64, 1 / 64))
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
            result["decode_mtp"]["fp8_cache"] = {
                "ms_decode": round(mf_ms, 4), "ms_decode_median": round(float(np.median(mfks)), 4),
                "kv_bytes": m_kv_bytes // 2,
                "achieved": round(m_kv_bytes / 2 / (mf_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                "speedup_vs_bf16_cache": round(m_ms / mf_ms, 3),
                "note": "inkattn_relattn_decode_fp8 on the same workload (E4M3 codes, scales 1/64)",
            }
            del mf, mcase8

    # ---------------- FP8 (E4M3) KV cache: the 16K SWA decode step again
    if not args.no_decode and not args.no_fp8:
        fcase = synth.workload_case(dwl, seed=0, past_device="cuda")
        fd = DeviceCase(fcase, torch, fp8_scales=(1 / 64, 1 / 64))
        fd.setup_decode_mq(torch)
        f_bytes = kv_bytes // 2

        def fstep(ev):
            fd.sconv()
            if ev is not None:
                ev[0].record()
            fd.decode_fp8()
            if ev is not None:
                ev[1].record()

        print(f"[bench] decode {dwl.name} with an FP8 cache", file=sys.stderr, flush=True)
        steady_clocks(torch, fstep, args.steady_s)
        f8_ms_step, f8ks = time_region(torch, fstep, None, d_steps, args.warmup)
        f8_ms = sum(f8ks) / len(f8ks)
        f8_gbs = f_bytes / (f8_ms * 1e-3) / 1e9
        result["decode_fp8"] = {
            "workload": dwl.name + " with an E4M3 KV cache (scales 1/64)",
            "ms_per_step": round(f8_ms_step, 4), "ms_decode": round(f8_ms, 4),
            "ms_decode_median": round(float(np.median(f8ks)), 4),
            "num_splits": fd.num_splits, "kv_bytes": f_bytes,
            "achieved": round(f8_gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac": round(f8_gbs / PEAK_HBM_GBS, 4),
            "speedup_vs_bf16_cache": round(d_ms / f8_ms, 3),
            "traffic": recorded_traffic(
                "decode_split_fp8_swa_decode_16k.traffic.txt",
                ["attention_sconv_amd/csrc/decode.hip",
                 "attention_sconv_amd/csrc/device_common.h"]),
            "note": "inkattn_sconv_fp8 + inkattn_relattn_decode_fp8; bytes = the E4M3 K+V "
                    "in the attended range",
        }
        del fd
        torch.cuda.empty_cache()

    import attention_sconv_amd as ink
    # ---------------- sconv of a plain activation (attention / MoE output)
    if not args.no_sconv_out:
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
    result["roofline"]["frac_of_measured"] = round(achieved / ceil["mfma_bf16_tflops"], 4)
    if "decode" in result:
        result["decode"]["frac_of_measured"] = round(gbs / ceil["hbm_read_gbs"], 4)

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case)

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
