"""CPU oracle for KV-outer block-sparse paged attention (test infrastructure).

This package is test infrastructure. Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it; the GPU library
never does, and it never imports the GPU library. The two share no code.
The only module both sides use is ``workloads`` (seeded input draws).

What it computes, and the passages it follows (alice-llm 2.0.0,
``src/sparse_attention``):

* ``index_ref.build_index_ref``: the CSR inverted index described by
  ``KvOuterIndex`` (types.rs). The builder itself is not on the pages. The
  loop here is the plainest reading of the index's field docs, and it is
  the spec that the GPU index must match bit-exactly.
* ``attention_ref.attention_qo_ref``: query-outer attention. For each query
  and KV head, dense softmax over the union of the tokens in its selected
  blocks, in float64. What a token contributes follows
  ``process_work_unit`` (forward.rs).
* ``kvouter_ref.forward_partials_ref`` / ``combine_ref``: the KV-outer partials
  ``(o, m, l)`` per edge and GQA lane (forward.rs, the ``ForwardPartials``
  field docs), each one block's share of the query-outer softmax, and their
  log-sum-exp merge. The pages name the combine pass (forward.rs, module doc)
  and say it is the log-sum-exp merge of FlashAttention, without its
  formula.
* ``dense_ref.dense_masked_ref``: brute-force masked dense attention over
  every logical position. It has no union gather and serves as a pin.
* ``kv16_ref.decode_kv16``: the float32 value of a K/V page word stored as
  bfloat16 or IEEE binary16 (not on the pages, which store fp32; attention
  on such pages is the fp32 oracle on the decoded values).

Pins live in ``tests/test_oracle_*.py`` (``-m "not gpu"``). No function here
is "parity unpinned".
"""
from .errors import SparseAttentionError
from .index_ref import build_index_ref, validate_build_inputs, batch_of, resolve_kv_lens
from .attention_ref import attention_qo_ref
from .kvouter_ref import forward_partials_ref, combine_ref
from .dense_ref import dense_masked_ref
from .kv16_ref import decode_bf16, decode_fp16, decode_kv16

__all__ = [
    "SparseAttentionError",
    "build_index_ref",
    "validate_build_inputs",
    "batch_of",
    "resolve_kv_lens",
    "attention_qo_ref",
    "forward_partials_ref",
    "combine_ref",
    "dense_masked_ref",
]
