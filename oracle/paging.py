"""Paged KV cache addressing -- fp64 oracle.

Test infrastructure only (see ``oracle/__init__.py``).

Source: the MI355X launch commands on the vLLM recipe pages
"thinkingmachines/Inkling" (*Client Usage*) and "thinkingmachines/Inkling-Small"
(*Client Usage*) run the model with a KV-cache block size of 128 tokens.

A sequence's token at logical position ``pos`` lives in physical slot
``block_table[pos // 128] * 128 + pos % 128``.  The oracle keeps the cache as
one float64 array indexed by slot, ``[num_slots, Hkv, d]``; how a GPU library
lays those slots out in memory is its own business, and tests translate.
"""

import numpy as np

BLOCK = 128


def slot_of(block_table_row, pos):
    """Physical slot of logical position ``pos`` of one sequence."""
    return int(block_table_row[pos // BLOCK]) * BLOCK + pos % BLOCK


def slots_for(block_table_row, positions):
    """Vector form of :func:`slot_of`."""
    positions = np.asarray(positions, dtype=np.int64)
    table = np.asarray(block_table_row, dtype=np.int64)
    return table[positions // BLOCK] * BLOCK + positions % BLOCK


class PagedStore:
    """A KV cache as a flat slot-indexed float64 array."""

    def __init__(self, num_blocks, num_kv_heads, head_dim):
        self.k = np.zeros((num_blocks * BLOCK, num_kv_heads, head_dim))
        self.v = np.zeros((num_blocks * BLOCK, num_kv_heads, head_dim))

    def write(self, slots, k_rows, v_rows):
        """Store rows [n, Hkv, d] at the given slots."""
        self.k[np.asarray(slots)] = k_rows
        self.v[np.asarray(slots)] = v_rows

    def gather(self, block_table_row, length):
        """Keys and values of positions 0..length-1 of one sequence."""
        s = slots_for(block_table_row, np.arange(length))
        return self.k[s], self.v[s]
