"""Plain fp64 CPU oracle for the Inkling attention-block hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The product package
(``attention_sconv_amd``) never imports it, and nothing here imports the
product: the two share no kernels, headers, helpers, tables or constants.  The
only module both sides use is ``synth`` (seeded synthetic inputs), which holds
none of the method's arithmetic.

What is computed, and where it comes from (page titles as headed on the web
pages this library is built from):

* ``sconv``      -- window-4 causal depthwise short convolution over key and
  value channels with a cache of the last three pre-convolution tokens
  ("vLLM, TML Inkling Day-0 support" news article, sections *Model
  Architecture / Sconv* and *Managing the sconv cache*).
* ``paging``     -- logical token position to physical KV-cache slot through a
  block table, block size 128 (vLLM recipe pages "thinkingmachines/Inkling"
  and "thinkingmachines/Inkling-Small", the MI355X launch commands).
* ``attention``  -- grouped-query attention, head size 128, sliding-window or
  full causal, with a learned relative-position term added to the
  pre-softmax logits instead of RoPE (news article, *Model Architecture /
  Attention*; recipe "thinkingmachines/Inkling", *Guide / Overview*).  The
  pages leave the parametrisation of that term open; this oracle uses the
  plainest table form, ``bias[h][min(i - j, R - 1)]`` (one row per query head,
  distances clipped to the table length).  Also the log-sum-exp merge of
  attention over a partition of the keys, which the split-K decode relies on
  (news article, *FA4 with sheared bias*, where the number of KV splits is
  chosen per configuration).

* ``fp8``        -- the OCP E4M3 code of a scaled key or value and what a
  cached code reads back as, for an FP8 KV cache (news article, *Roadmap*:
  FP8 for the global-attention layers).  Attention over such a cache is the
  attention above on the read-back keys and values.  For FP8 matrix
  products: the per-tile query quantizer and, in ``attention``, the bound
  on what rounding the probabilities to E4M3 can move
  (``relattn_prefill_p8_bounds``).

Everything is evaluated in float64 straight from the definitions: no tiling,
no online softmax, no splits.  Inputs may be float32 or bfloat16-representable
values held in float32; they are upcast exactly.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines (torch float64 ``conv1d`` and
``scaled_dot_product_attention`` on the CPU, torch's ``float8_e4m3fn``), metamorphic invariants and a
pure-Python brute force.  No function is "parity unpinned".
"""

from .sconv import sconv_sequence, sconv_batch  # noqa: F401
from .paging import BLOCK, slot_of, slots_for, PagedStore  # noqa: F401
from .attention import (  # noqa: F401
    visible_key_range,
    relattn_rows,
    relattn_prefill,
    relattn_prefill_p8_bounds,
    relattn_decode,
    lse_merge,
)
from . import fp8  # noqa: F401
