"""Float64 CPU oracle for the paged-KV attention path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code with the HIP library; the two meet
only through the seeded inputs of ``workloads/``.

It is the plain definition, computed slowly: gather the pages of each request
into a contiguous sequence, build the full score matrix, mask it, take the
softmax, multiply by V. Sources (FlashInfer API pages):

* ``flashinfer.page.append_paged_kv_cache`` -- Parameters, Example, Note
  (append, ``get_seq_lens``, ``get_batch_indices_positions``);
* ``flashinfer.prefill.cudnn_batch_prefill_with_kv_cache`` -- Parameters,
  Returns, Note (batch prefill with causal mask, GQA, fp8 scales, LSE);
* ``flashinfer.decode.trtllm_batch_decode_with_kv_cache`` -- Parameters
  (block_tables decode, bmm1/bmm2 scales, window_left, sinks, q_len_per_req).

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: the arrays the append page prints, closed forms, library routines
(``torch.float8_e4m3fn``, ``scaled_dot_product_attention``) and brute force.
"""

from .formats import decode_bits, e4m3fn_table, encode_e4m3fn, bits_dtype
from .paging import (
    get_seq_lens,
    get_batch_indices_positions,
    csr_to_block_tables,
    append_paged_kv_cache,
    gather_pages,
)
from .attention import (
    allowed_mask,
    attention,
    batch_prefill,
    batch_prefill_ragged,
    batch_decode,
    allowed_pairs,
    keys_read,
)

__all__ = [
    "decode_bits",
    "e4m3fn_table",
    "bits_dtype",
    "get_seq_lens",
    "get_batch_indices_positions",
    "csr_to_block_tables",
    "append_paged_kv_cache",
    "gather_pages",
    "allowed_mask",
    "attention",
    "batch_prefill",
    "batch_decode",
    "allowed_pairs",
    "keys_read",
]
