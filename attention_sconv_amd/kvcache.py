"""Device-memory helpers for the library's paged KV-cache layout.

  k_cache [num_blocks][Hkv][128 tokens][128 dims]
  v_cache [num_blocks][Hkv][128 dims][128 tokens]   (V transposed per page)

A token at slot s = block * 128 + offset lives in k_cache[block, h, offset, :]
and v_cache[block, h, :, offset].  These helpers only allocate and re-view
memory; no attention arithmetic happens here.
"""

import torch

PAGE = 128
HEAD_DIM = 128


def torch_dtype(dtype):
    """Cache element type: bf16 / fp32, or "fp8" (E4M3 codes held as uint8)."""
    if dtype == "fp8":
        return torch.uint8
    return torch.bfloat16 if dtype in (1, "bf16") else torch.float32


def alloc(num_blocks, num_kv_heads, dtype, device="cuda"):
    td = torch_dtype(dtype)
    k = torch.empty((num_blocks, num_kv_heads, PAGE, HEAD_DIM), dtype=td, device=device)
    v = torch.empty((num_blocks, num_kv_heads, HEAD_DIM, PAGE), dtype=td, device=device)
    return k, v


def from_slots(k_slots, v_slots):
    """[num_slots, Hkv, d] slot-major tensors -> (k_cache, v_cache) in the
    library layout (new contiguous tensors on the same device)."""
    S, H, D = k_slots.shape
    nb = S // PAGE
    k = k_slots.reshape(nb, PAGE, H, D).permute(0, 2, 1, 3).contiguous()
    v = v_slots.reshape(nb, PAGE, H, D).permute(0, 2, 3, 1).contiguous()
    return k, v


def to_slots(k_cache, v_cache):
    """Inverse of :func:`from_slots`: (k_cache, v_cache) -> [num_slots, Hkv, d]."""
    nb, H, P, D = k_cache.shape
    k = k_cache.permute(0, 2, 1, 3).reshape(nb * P, H, D)
    v = v_cache.permute(0, 3, 1, 2).reshape(nb * P, H, D)
    return k, v


def slots_of(k_cache, v_cache, slots):
    """Rows of the given slots as [n, Hkv, d] tensors (K, V)."""
    slots = torch.as_tensor(slots, device=k_cache.device, dtype=torch.long)
    blk, off = slots // PAGE, slots % PAGE
    k = k_cache[blk, :, off, :]
    v = v_cache[blk, :, :, off]
    return k, v
