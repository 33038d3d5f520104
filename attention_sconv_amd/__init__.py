"""libinkattn for MI355X (gfx950): the Inkling attention-block hot path.

* ``inkattn_sconv``            -- window-4 short convolution of keys and values
                                 fused with the paged KV-cache write and the
                                 three-token state update;
* ``inkattn_sconv_paged``      -- the same with the sconv state kept in a paged
                                 cache (a window-3 virtual layer; prefix caching);
* ``inkattn_sconv_out``        -- the same convolution on a plain activation
                                 tensor (attention output, MoE output);
* ``inkattn_sconv_fp8``, ``inkattn_relattn_decode_fp8``,
  ``inkattn_relattn_prefill_fp8`` -- the sconv cache write, the (multi-query)
                                 decode and the prefill with an FP8 (OCP
                                 E4M3, scaled) KV cache;
* ``inkattn_relattn_prefill_fp8_mma`` -- the prefill over an E4M3 cache with
                                 FP8 matrix products (Q and P rounded to E4M3),
                                 for the global-attention layers;
* ``inkattn_relattn_prefill``  -- relative-position GQA attention over new
                                 tokens (bf16/fp32 MFMA, sheared bias band);
* ``inkattn_relattn_decode``   -- split-K paged decode plus log-sum-exp merge;
* ``inkattn_relattn_decode_noalloc`` -- the same with its split partials in a
                                 static device array (for callers that cannot
                                 allocate);
* ``inkattn_relattn_decode_mq`` -- the same for a few query tokens per sequence
                                 (verification of multi-token-prediction drafts).

``inkattn_probe_mfma_bf16`` and ``inkattn_probe_stream_read`` are diagnostics
(measured MFMA and HBM-read ceilings), not part of the attention path.

The functions mirror the C ABI in ``include/inkattn.h`` one to one and take
torch device tensors (torch supplies memory and streams only).  The helpers in
``kvcache`` allocate the cache in the library's layout.
"""

from ._lib import (  # noqa: F401
    BF16, FP32, OK, EINVAL, ENOTSUP, EHIP, ESCRATCH, EXPORTED, LIB_PATH, NOALLOC_SCRATCH_BYTES,
    AttnDesc, InkattnError, make_desc, status_string,
    inkattn_sconv, inkattn_relattn_prefill, inkattn_relattn_decode,
    inkattn_relattn_decode_noalloc,
    inkattn_relattn_decode_num_splits, inkattn_relattn_decode_workspace_size,
    inkattn_sconv_paged, inkattn_sconv_out, inkattn_sconv_fp8, inkattn_relattn_decode_fp8,
    inkattn_relattn_decode_mq, inkattn_relattn_decode_mq_num_splits,
    inkattn_relattn_decode_mq_workspace_size,
    inkattn_relattn_prefill_fp8, inkattn_relattn_prefill_fp8_workspace_size,
    inkattn_relattn_prefill_fp8_mma,
    inkattn_probe_mfma_bf16, inkattn_probe_stream_read,
    PROBE_MFMA_WAVES, PROBE_MFMA_CHAINS, PROBE_READ_GROUPS,
)
from . import kvcache  # noqa: F401
