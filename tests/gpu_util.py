"""Host-side helpers for the GPU parity tests: move a ``synth`` case to the
device, call the library through its C ABI, and build the oracle's view of
the same inputs.  No attention arithmetic here: expected values come from
``oracle`` only."""

import numpy as np
import torch

import attention_sconv_amd as ink
from attention_sconv_amd import kvcache
import oracle

from parity import TOL, check_attention, check_close, check_lse, check_out  # noqa: F401


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def ddtype(dtype):
    return ink.BF16 if dtype == "bf16" else ink.FP32


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdtype(dtype))


def idev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def fp8_codes(x, scale):
    """E4M3 codes of x / scale (saturated) through torch's float8_e4m3fn cast:
    how the tests draw the cached context of an FP8 cache (an input)."""
    return (x.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


FP8_NAN = 0x7F          # an E4M3 NaN code, for cache slots nothing wrote


class GpuCase:
    """Device copies of a synth.Case plus a KV cache in the library layout.
    Cache slots that no token has written hold NaN, so any read of them shows.
    With ``fp8_scales=(k_scale, v_scale)`` the cache holds E4M3 codes; the
    cached context is the synth draw cast to E4M3 (``past_codes``)."""

    def __init__(self, case, fill_nan=True, fp8_scales=None):
        self.case = c = case
        self.dt = c.dtype
        self.fp8 = fp8_scales
        self.past_codes = None
        self.q = dev(c.q, c.dtype)
        self.k_pre = dev(c.k_pre, c.dtype)
        self.v_pre = dev(c.v_pre, c.dtype)
        self.conv_w = dev(c.conv_w, c.dtype)
        self.conv_state = dev(c.conv_state, c.dtype)
        self.state_slot = idev(c.state_slot)
        self.cu = idev(c.cu_seqlens)
        self.slot_mapping = idev(c.slot_mapping)
        self.block_table = idev(c.block_table)
        self.seq_lens = idev(c.seq_lens)
        self.bias = dev(c.bias, c.dtype)
        nan = FP8_NAN if fp8_scales else float("nan")
        if c.past_k is not None:
            pk = c.past_k if torch.is_tensor(c.past_k) else dev(c.past_k, c.dtype)
            pv = c.past_v if torch.is_tensor(c.past_v) else dev(c.past_v, c.dtype)
            if fp8_scales:
                pk = fp8_codes(pk, fp8_scales[0])
                pv = fp8_codes(pv, fp8_scales[1])
                self.past_codes = (pk, pv)
            self.k_cache, self.v_cache = kvcache.from_slots(pk, pv)
            if fill_nan:
                # slots beyond each sequence's context are unwritten
                self._nan_unwritten(nan)
        else:
            self.k_cache, self.v_cache = kvcache.alloc(c.num_blocks, c.num_kv_heads,
                                                       "fp8" if fp8_scales else c.dtype)
            if fill_nan:
                self.k_cache.fill_(nan)
                self.v_cache.fill_(nan)
            else:
                self.k_cache.zero_()
                self.v_cache.zero_()

    def _nan_unwritten(self, nan=float("nan")):
        c = self.case
        written = np.zeros(c.num_blocks * 128, dtype=bool)
        for b in range(len(c.seq_lens)):
            pos = np.arange(int(c.ctx_lens[b]))
            written[oracle.slots_for(c.block_table[b], pos)] = True
        bad = torch.from_numpy(np.nonzero(~written)[0]).to("cuda")
        blk, off = bad // 128, bad % 128
        self.k_cache[blk, :, off, :] = nan
        self.v_cache[blk, :, :, off] = nan

    # ---- library calls (through the C ABI) ----
    def sconv(self, stream=None):
        c = self.case
        if self.fp8:
            ink.inkattn_sconv_fp8(ddtype(self.dt), c.num_kv_heads, 128, len(c.q_lens),
                                  c.num_tokens, int(c.q_lens.max()), self.k_pre, self.v_pre,
                                  self.conv_w, self.conv_state, self.state_slot, self.cu,
                                  self.slot_mapping, self.fp8[0], self.fp8[1], self.k_cache,
                                  self.v_cache, stream)
            return
        ink.inkattn_sconv(ddtype(self.dt), c.num_kv_heads, 128, len(c.q_lens), c.num_tokens,
                          int(c.q_lens.max()), self.k_pre, self.v_pre, self.conv_w,
                          self.conv_state, self.state_slot, self.cu, self.slot_mapping,
                          self.k_cache, self.v_cache, stream)

    def desc(self):
        c = self.case
        return ink.make_desc(ddtype(self.dt), c.num_q_heads, c.num_kv_heads, c.window,
                             c.bias_len)

    def prefill(self, with_lse=True, stream=None):
        c = self.case
        out = torch.empty_like(self.q)
        lse = (torch.empty((c.num_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_prefill(self.desc(), len(c.q_lens), c.num_tokens,
                                    int(c.q_lens.max()), self.q, self.k_cache, self.v_cache,
                                    self.block_table, self.block_table.shape[1], self.cu,
                                    self.seq_lens, self.bias, out, lse, stream)
        return out, lse

    def decode(self, num_splits=0, with_lse=True, stream=None):
        c = self.case
        assert (c.q_lens == 1).all()
        B = len(c.q_lens)
        d = self.desc()
        L = int(c.seq_lens.max())
        ws_bytes = ink.inkattn_relattn_decode_workspace_size(d, B, L, num_splits)
        ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
        out = torch.empty_like(self.q)
        lse = (torch.empty((B, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_decode(d, B, L, self.q, self.k_cache, self.v_cache,
                                   self.block_table, self.block_table.shape[1], self.seq_lens,
                                   self.bias, out, lse, num_splits, ws, ws_bytes, stream)
        return out, lse


    def decode_fp8(self, num_splits=0, with_lse=True, stream=None):
        """inkattn_relattn_decode_fp8 over all new tokens of every sequence."""
        c = self.case
        B = len(c.q_lens)
        d = self.desc()
        L = int(c.seq_lens.max())
        Q = int(c.q_lens.max())
        ws_bytes = ink.inkattn_relattn_decode_mq_workspace_size(d, B, c.num_tokens, Q, L,
                                                                num_splits)
        ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
        out = torch.empty_like(self.q)
        lse = (torch.empty((c.num_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_decode_fp8(d, B, c.num_tokens, Q, L, self.q, self.k_cache,
                                       self.v_cache, self.fp8[0], self.fp8[1], self.block_table,
                                       self.block_table.shape[1], self.cu, self.seq_lens,
                                       self.bias, out, lse, num_splits, ws, ws_bytes, stream)
        return out, lse

    def prefill_fp8(self, with_lse=True, stream=None):
        """inkattn_relattn_prefill_fp8 over all new tokens of every sequence."""
        c = self.case
        B = len(c.q_lens)
        d = self.desc()
        mb = self.block_table.shape[1]
        ws_bytes = ink.inkattn_relattn_prefill_fp8_workspace_size(d, B, mb)
        ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
        ws.fill_(float("nan"))      # nothing may read a page the call did not write
        out = torch.empty_like(self.q)
        lse = (torch.empty((c.num_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_prefill_fp8(d, B, c.num_tokens, int(c.q_lens.max()), self.q,
                                        self.k_cache, self.v_cache, self.fp8[0], self.fp8[1],
                                        self.block_table, mb, self.cu, self.seq_lens, self.bias,
                                        out, lse, ws, ws_bytes, stream)
        return out, lse

    def prefill_fp8_mma(self, with_lse=True, stream=None):
        """inkattn_relattn_prefill_fp8_mma over all new tokens of every sequence."""
        c = self.case
        B = len(c.q_lens)
        d = self.desc()
        mb = self.block_table.shape[1]
        out = torch.empty_like(self.q)
        lse = (torch.empty((c.num_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_prefill_fp8_mma(d, B, c.num_tokens, int(c.q_lens.max()), self.q,
                                            self.k_cache, self.v_cache, self.fp8[0],
                                            self.fp8[1], self.block_table, mb, self.cu,
                                            self.seq_lens, self.bias, out, lse, stream)
        return out, lse

    def decode_mq(self, num_splits=0, with_lse=True, stream=None):
        """All new tokens of every sequence in one multi-query decode call."""
        c = self.case
        B = len(c.q_lens)
        d = self.desc()
        L = int(c.seq_lens.max())
        Q = int(c.q_lens.max())
        ws_bytes = ink.inkattn_relattn_decode_mq_workspace_size(d, B, c.num_tokens, Q, L,
                                                                num_splits)
        ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
        out = torch.empty_like(self.q)
        lse = (torch.empty((c.num_tokens, c.num_q_heads), dtype=torch.float32, device="cuda")
               if with_lse else None)
        ink.inkattn_relattn_decode_mq(d, B, c.num_tokens, Q, L, self.q, self.k_cache,
                                      self.v_cache, self.block_table, self.block_table.shape[1],
                                      self.cu, self.seq_lens, self.bias, out, lse, num_splits,
                                      ws, ws_bytes, stream)
        return out, lse


# ---- oracle side ----
def oracle_sconv(case):
    return oracle.sconv_batch(case.k_pre, case.v_pre, case.conv_w, case.conv_state,
                              case.state_slot, case.cu_seqlens)


def oracle_kv(case, b, k_new, v_new, lo=0, fp8=None):
    """Logical K, V [L, Hkv, d] (float64) of sequence b: cached context from
    the synth draw, then the oracle's post-convolution rows of the new tokens.
    Positions below ``lo`` (outside every query's window) are left at zero.
    With ``fp8=(gpu_case, k_scale, v_scale)``: the context read back from
    the cached codes and the new rows through the oracle's E4M3 quantizer."""
    if fp8 is not None:
        return _oracle_kv_fp8(case, b, k_new, v_new, lo, *fp8)
    c = case
    H, d = c.num_kv_heads, 128
    ctx, L = int(c.ctx_lens[b]), int(c.seq_lens[b])
    K = np.zeros((L, H, d))
    V = np.zeros((L, H, d))
    if ctx > lo:
        slots = oracle.slots_for(c.block_table[b], np.arange(lo, ctx))
        pk, pv = c.past_k, c.past_v
        if torch.is_tensor(pk):
            idx = torch.from_numpy(slots).to(pk.device)
            K[lo:ctx] = pk[idx].float().cpu().numpy()
            V[lo:ctx] = pv[idx].float().cpu().numpy()
        else:
            K[lo:ctx] = pk[slots]
            V[lo:ctx] = pv[slots]
    t0, t1 = int(c.cu_seqlens[b]), int(c.cu_seqlens[b + 1])
    K[ctx:] = k_new[t0:t1].reshape(-1, H, d)
    V[ctx:] = v_new[t0:t1].reshape(-1, H, d)
    return K, V


def _oracle_kv_fp8(case, b, k_new, v_new, lo, gc, ks, vs):
    c = case
    H, d = c.num_kv_heads, 128
    ctx, L = int(c.ctx_lens[b]), int(c.seq_lens[b])
    K = np.zeros((L, H, d))
    V = np.zeros((L, H, d))
    if ctx > lo:
        slots = oracle.slots_for(c.block_table[b], np.arange(lo, ctx))
        idx = torch.from_numpy(slots).to(gc.past_codes[0].device)
        K[lo:ctx] = oracle.fp8.dequantize(gc.past_codes[0][idx].cpu().numpy(), ks)
        V[lo:ctx] = oracle.fp8.dequantize(gc.past_codes[1][idx].cpu().numpy(), vs)
    t0, t1 = int(c.cu_seqlens[b]), int(c.cu_seqlens[b + 1])
    K[ctx:] = oracle.fp8.dequantize(oracle.fp8.quantize(k_new[t0:t1], ks), ks).reshape(-1, H, d)
    V[ctx:] = oracle.fp8.dequantize(oracle.fp8.quantize(v_new[t0:t1], vs), vs).reshape(-1, H, d)
    return K, V


def assert_close(got, want, tol, what="", relative=False):
    """max |got - want| <= tol, or, with ``relative``, <= tol * max(1, |want|)."""
    return check_close(got, want, tol, what, relative)


def assert_parity(got, want, dtype, what=""):
    """Elementwise output bound of the storage dtype (see ``parity``)."""
    return check_out(got, want, dtype, what)


def assert_lse(got, want, dtype, what="lse"):
    """Absolute lse bound of the storage dtype (see ``parity``)."""
    return check_lse(got, want, dtype, what)


def assert_attention(got_o, want_o, got_l, want_l, dtype, what="", scale_aware=False):
    """Output and lse bounds; ``scale_aware`` adds the per-row bf16 bound for
    workloads whose outputs are far below unit scale (see ``parity``)."""
    return check_attention(got_o, want_o, got_l, want_l, dtype, what, scale_aware)
