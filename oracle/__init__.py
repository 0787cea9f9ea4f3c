"""Float64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP product path
never calls it, and this package never imports the product package: the two
share no code.  Inputs reach both sides from ``workloads`` (seeded generators
that hold no attention arithmetic).

Two independent implementations of the same result:

* ``naive.attention_naive`` / ``naive.attention_rows`` -- the plain definition
  softmax(scale * Q K^T) V with an optional causal mask, two-pass stable
  softmax over each full row, plus the per-row logsumexp L.
* ``gqa.attention_gqa`` -- grouped-query attention: each K/V head serves a
  group of consecutive query heads; the plain definition applied per query
  head against its group's K/V.
* ``backward.attention_backward`` -- dQ, dK, dV of the scalar loss sum(dO * O),
  the chain rule of the plain definition written out (with grouped K/V heads);
  ``dq_rows`` / ``dkdv_cols`` restrict it to chosen query rows or keys.
* ``decode.attention_decode`` -- N_q queries (the last N_q positions) against
  N_k keys, and ``decode.merge_partials``, the logsumexp merge of attention
  partials over disjoint key ranges.
* ``masks.attention_alibi`` / ``masks.attention_blocksparse`` -- the plain
  definition with ALiBi linear biases or a block-sparse mask.
* ``online.attention_online`` -- the blockwise online-softmax recurrence
  (running row max m, running row sum l, rescale of the partial output when m
  grows, one normalisation at the end), for any block sizes.

The pages state the blockwise method reaches the identical (exact) result, so
the two must agree to float64 rounding.  Pins: see ``tests/test_oracle_pins.py``.
Every function here is pinned; none is "parity unpinned".
"""

from .naive import attention_naive, attention_rows
from .gqa import attention_gqa, expand_kv
from .online import attention_online
from .backward import attention_backward, backward_head, delta_rows, dkdv_cols, dq_rows
from .decode import attention_decode, attention_decode_gqa, merge_partials, partial_over_keys
from .masks import attention_alibi, attention_biased, attention_blocksparse, expand_block_mask
from .compare import errors

__all__ = ["attention_naive", "attention_rows", "attention_gqa", "expand_kv", "attention_online",
           "attention_backward", "backward_head", "delta_rows", "dq_rows", "dkdv_cols",
           "attention_decode", "attention_decode_gqa", "partial_over_keys", "merge_partials",
           "attention_alibi", "attention_biased", "attention_blocksparse", "expand_block_mask", "errors"]
