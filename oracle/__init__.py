"""CPU fp64 oracle for load-balanced context-parallel causal attention and GQA decode.

TEST INFRASTRUCTURE ONLY. This package is the slow, plainly written reference that the
HIP path is checked against. Only the test suite, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import it. The product library never calls
it, and it shares no code, tables or helpers with the HIP sources.

Sources (web pages, cited by title and section):

* "Add context parallelism" (MaxText PR 1445), Description: context parallelism
  all-gathers keys/values and shards queries along the sequence; tokens *and the attention
  mask* are reordered for load balance, with the cp=2 example giving one device tokens
  0,1,6,7 and the other 2,3,4,5.
* "Add support for EP to context parallelism in self-attention" (MaxText PR 2023),
  Description / unit test: the sharded result is compared against un-sharded dot-product
  attention (the role this oracle plays), with and without load balancing, for MHA and MLA.
* "Add Pallas GPU decode attention in Maxtext inference" (MaxText PR 1066), Description /
  Tests: grouped-query single-token decode attention over a KV cache filled to the current
  length.
* "rename context to context_autoregressive" (MaxText PR 1453), Description: inference
  context parallelism splits the cache along its length (merge of per-slice decodes), and the
  decode benchmark quantizes the KV cache to int8 (``oracle.quant``: the absmax per-row
  reading taken for it).
* "Add context parallelism" (MaxText PR 1445), Description, again for the backward pass
  (``oracle.backward``): the shard's gradients by the chain rule through the forward above.

Every function computes in float64 from inputs upcast exactly from their stored dtype.

Parity status: every function here is pinned by ``tests/test_oracle.py`` (worked example
printed on the pages, brute force, a library routine, closed forms and invariants). No
function is "parity unpinned".
"""

from .lb_index import (
    load_balance_perm,
    inverse_perm,
    shard_row_range,
    shard_positions,
    causal_pair_count,
    contiguous_shard_positions,
)
from .attention import (
    causal_attention_ref,
    cp_attention_ref,
    decode_ref,
    decode_merge_ref,
    permute_ref,
    unpermute_ref,
)
from .quant import kv_quantize_ref, dequantize_ref, decode_int8_ref
from .backward import causal_attention_bwd_ref, cp_attention_bwd_ref

__all__ = [
    "load_balance_perm",
    "inverse_perm",
    "shard_row_range",
    "shard_positions",
    "causal_pair_count",
    "contiguous_shard_positions",
    "causal_attention_ref",
    "cp_attention_ref",
    "decode_ref",
    "decode_merge_ref",
    "kv_quantize_ref",
    "dequantize_ref",
    "decode_int8_ref",
    "causal_attention_bwd_ref",
    "cp_attention_bwd_ref",
    "permute_ref",
    "unpermute_ref",
]
