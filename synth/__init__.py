"""Seeded synthetic inputs for the attention-block hot path.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__`` and
feeds both the GPU library and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers, rounds them to the storage dtype and
lays out the integer bookkeeping (sequence offsets, block tables, slot
numbers) that a serving engine would hand to the kernels.

Recipe (fixed draw order from one ``numpy.random.Generator(PCG64(seed))``):

  q, k_pre, v_pre      N(0, 1)
  w_k, w_v             N(0, 0.5^2)   (std 0.5: four taps of unit inputs give
                                       post-convolution values of unit scale)
  bias                 N(0, 1)
  conv_state           N(0, 1) for sequences with earlier context, else 0
  past K / V           N(0, 1)       (post-convolution cache of earlier tokens)
  block permutation    random permutation of the block pool

bfloat16 inputs are rounded from the float32 draws to nearest-even and kept as
float32 arrays holding bfloat16-representable values, so the same numbers
reach the GPU (exact conversion) and the oracle (exact upcast).  Past K/V of a
large pool may instead be drawn by ``torch`` on a given device (seeded
``torch.Generator``); the oracle then reads the slots it needs back.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 128
HEAD_DIM = 128


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  NaN/Inf are not expected in synthetic data."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _draw(rng, shape, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration (shapes only)."""
    name: str
    kind: str            # "prefill" or "decode"
    dtype: str           # "fp32" or "bf16"
    batch: int
    seq_len: int         # keys per sequence including the new tokens
    q_len: int           # new tokens per sequence (= seq_len for prefill)
    num_q_heads: int
    num_kv_heads: int
    window: int          # 0 = full causal
    bias_len: int        # R
    head_dim: int = HEAD_DIM
    description: str = ""


WORKLOADS = {
    "tiny_fp32_swa_prefill": Workload(
        "tiny_fp32_swa_prefill", "prefill", "fp32", 1, 256, 256, 4, 1, 64, 64,
        description="1 seq, T=256, Hq=4, Hkv=1, window 64, R=64, fp32"),
    "swa_prefill_8k": Workload(
        "swa_prefill_8k", "prefill", "bf16", 1, 8192, 8192, 32, 4, 2048, 2048,
        description="batch 1, T=8192, Hq=32, Hkv=4, window 2048, R=2048, bf16"),
    "full_prefill_32k": Workload(
        "full_prefill_32k", "prefill", "bf16", 2, 32768, 32768, 32, 4, 0, 32768,
        description="batch 2, T=32768, Hq=32, Hkv=4, full causal, R=32768, bf16"),
    "swa_decode_16k": Workload(
        "swa_decode_16k", "decode", "bf16", 64, 16384, 1, 32, 4, 4096, 4096,
        description="batch 64, L=16384, window 4096, R=4096, Hq=32, Hkv=4, bf16"),
    "swa_decode_16k_mtp9": Workload(
        "swa_decode_16k_mtp9", "decode", "bf16", 64, 16384, 9, 32, 4, 4096, 4096,
        description="batch 64, L=16384 with the last 9 tokens (1 accepted + 8 MTP drafts) "
                    "as queries, window 4096, R=4096, Hq=32, Hkv=4, bf16"),
    "full_decode_1m": Workload(
        "full_decode_1m", "decode", "bf16", 4, 1048576, 1, 32, 4, 0, 1048576,
        description="batch 4, L=1,048,576, full causal, R=1,048,576, Hq=32, "
                    "Hkv=4, bf16"),
}


@dataclass
class Case:
    """All inputs of one call sequence (sconv, then attention).

    Arrays are numpy unless ``past_device`` was given, in which case
    ``past_k`` / ``past_v`` are torch tensors on that device.
    """
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    window: int
    bias_len: int
    q_lens: np.ndarray        # [B] new tokens per sequence
    ctx_lens: np.ndarray      # [B] tokens already cached per sequence
    seq_lens: np.ndarray      # [B] = ctx + q
    cu_seqlens: np.ndarray    # [B+1] offsets of the new tokens
    q: np.ndarray             # [N, Hq, d]
    k_pre: np.ndarray         # [N, Hkv*d]
    v_pre: np.ndarray         # [N, Hkv*d]
    conv_w: np.ndarray        # [2, Hkv*d, 4]
    bias: np.ndarray          # [Hq, R]
    conv_state: np.ndarray    # [B, 2, 3, Hkv*d]   (row b = sequence b)
    state_slot: np.ndarray    # [B]
    num_blocks: int
    block_table: np.ndarray   # [B, max_blocks]  int32
    slot_mapping: np.ndarray  # [N] int32, slot of each new token
    past_k: object = None     # [num_blocks*128, Hkv, d] post-conv, or None
    past_v: object = None
    head_dim: int = HEAD_DIM
    extra: dict = field(default_factory=dict)

    @property
    def num_tokens(self):
        return int(self.cu_seqlens[-1])

    @property
    def channels(self):
        return self.num_kv_heads * self.head_dim


def make_case(dtype, q_lens, ctx_lens, num_q_heads, num_kv_heads, window,
              bias_len, seed=0, extra_blocks=0, past_device: Optional[str] = None,
              shuffle_state_slots=False):
    """Draw one case.  ``q_lens[b]`` new tokens follow ``ctx_lens[b]`` cached
    tokens in sequence b.  Cached tokens get random post-convolution K/V and
    the sequence a random pre-convolution state; fresh sequences (ctx 0) get a
    zero state and no past K/V."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    B = len(q_lens)
    d = HEAD_DIM
    C = num_kv_heads * d
    seq_lens = q_lens + ctx_lens
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(q_lens)
    N = int(cu[-1])

    q = _draw(rng, (N, num_q_heads, d), 1.0, dtype)
    k_pre = _draw(rng, (N, C), 1.0, dtype)
    v_pre = _draw(rng, (N, C), 1.0, dtype)
    w_k = _draw(rng, (C, 4), 0.5, dtype)
    w_v = _draw(rng, (C, 4), 0.5, dtype)
    bias = _draw(rng, (num_q_heads, bias_len), 1.0, dtype)
    state = _draw(rng, (B, 2, 3, C), 1.0, dtype)
    state[ctx_lens == 0] = 0.0

    blocks_per_seq = (seq_lens + BLOCK - 1) // BLOCK
    num_blocks = int(blocks_per_seq.sum()) + int(extra_blocks)
    num_slots = num_blocks * BLOCK
    past_k = past_v = None
    if int(ctx_lens.max(initial=0)) > 0:
        if past_device is None:
            past_k = _draw(rng, (num_slots, num_kv_heads, d), 1.0, dtype)
            past_v = _draw(rng, (num_slots, num_kv_heads, d), 1.0, dtype)
        else:
            import torch
            g = torch.Generator(device=past_device)
            g.manual_seed(int(rng.integers(0, 2**62)))
            tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
            shape = (num_slots, num_kv_heads, d)
            past_k = torch.randn(shape, generator=g, device=past_device,
                                 dtype=torch.float32).to(tdt)
            past_v = torch.randn(shape, generator=g, device=past_device,
                                 dtype=torch.float32).to(tdt)

    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = int(blocks_per_seq.max(initial=1))
    table = np.zeros((B, max(max_blocks, 1)), dtype=np.int32)
    off = 0
    for b in range(B):
        nb = int(blocks_per_seq[b])
        table[b, :nb] = perm[off:off + nb]
        off += nb
    slot_mapping = np.zeros(N, dtype=np.int32)
    for b in range(B):
        pos = np.arange(ctx_lens[b], seq_lens[b])
        slot_mapping[cu[b]:cu[b + 1]] = table[b, pos // BLOCK] * BLOCK + pos % BLOCK
    state_slot = np.arange(B, dtype=np.int32)
    if shuffle_state_slots:
        state_slot = rng.permutation(B).astype(np.int32)
        state = state[np.argsort(state_slot)]
    return Case(dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                window=window, bias_len=bias_len, q_lens=q_lens, ctx_lens=ctx_lens,
                seq_lens=seq_lens, cu_seqlens=cu, q=q, k_pre=k_pre, v_pre=v_pre,
                conv_w=np.stack([w_k, w_v]), bias=bias, conv_state=state,
                state_slot=state_slot, num_blocks=num_blocks, block_table=table,
                slot_mapping=slot_mapping, past_k=past_k, past_v=past_v)


def workload_case(wl: Workload, seed=0, past_device=None, batch=None):
    """The case for a named workload (optionally with fewer sequences)."""
    B = wl.batch if batch is None else batch
    if wl.kind == "prefill":
        return make_case(wl.dtype, [wl.q_len] * B, [wl.seq_len - wl.q_len] * B,
                         wl.num_q_heads, wl.num_kv_heads, wl.window, wl.bias_len,
                         seed=seed, past_device=past_device)
    return make_case(wl.dtype, [wl.q_len] * B, [wl.seq_len - wl.q_len] * B, wl.num_q_heads,
                     wl.num_kv_heads, wl.window, wl.bias_len, seed=seed,
                     past_device=past_device)


@dataclass
class SconvOutCase:
    """Inputs of the short convolution on a plain activation tensor."""
    dtype: str
    x: np.ndarray            # [N, C]
    conv_w: np.ndarray       # [C, 4]
    conv_state: np.ndarray   # [num_slots, 3, C]
    state_slot: np.ndarray   # [B] int32, distinct
    cu_seqlens: np.ndarray   # [B + 1] int64
    q_lens: np.ndarray       # [B]


def make_sconv_out_case(dtype, q_lens, channels, seed=0, extra_slots=2, fresh=None):
    """Ragged chunks of a [tokens][channels] activation, per-channel taps and a
    state table with ``extra_slots`` rows no sequence owns.  ``fresh[b]`` (all
    False by default) gives sequence b a zero state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    B = len(q_lens)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(q_lens)
    x = _draw(rng, (int(cu[-1]), channels), 1.0, dtype)
    w = _draw(rng, (channels, 4), 0.5, dtype)
    slots = B + int(extra_slots)
    state = _draw(rng, (slots, 3, channels), 1.0, dtype)
    state_slot = rng.permutation(slots)[:B].astype(np.int32)
    if fresh is not None:
        for b in range(B):
            if fresh[b]:
                state[state_slot[b]] = 0.0
    return SconvOutCase(dtype=dtype, x=x, conv_w=w, conv_state=state, state_slot=state_slot,
                        cu_seqlens=cu, q_lens=q_lens)
