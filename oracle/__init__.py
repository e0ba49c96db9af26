"""fp64 CPU oracle for per-rank context-parallel attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (no kernels, headers, helpers or constants); both sides receive the
same seeded inputs from the workload generator, which holds none of the
method's arithmetic.

What it computes, plainly and slowly, in float64 numpy:

* ``attention`` -- softmax(Q K^T * scale) V with an explicit log-sum-exp, the
  semantics of the unmasked, non-causal, dropout-free
  ``scaled_dot_product_attention`` call in the ParaAttention README section
  "Run Unified Attention (Hybird Ulysses Style and Ring Style) with
  torch.compile";
* ``lse_merge`` -- combining two partial (output, LSE) pairs by log-sum-exp
  rescaling, the fp32 ring numerics named by ``convert_to_fp32`` in the
  ``ContextParallelConfig`` parameters ("Parallelism" API page);
* ``ring_attention`` -- the ring loop: attention of the local Q against each
  K/V chunk in turn, merged in chunk order ("Context parallelism" page, Ring
  Attention and Ring Anything Attention sections);
* ``ulysses_seq_to_head`` / ``ulysses_head_to_seq`` -- the Ulysses regroup from
  sequence shards holding all heads to head groups holding the whole sequence,
  and back ("Context parallelism" page, Ulysses Attention section);
* ``anything_seq_to_head`` / ``anything_head_to_seq`` -- the same regroup with
  uneven sequence shards and head groups (Ulysses Anything Attention section);
* ``unified_rank_share`` / ``unified_all_ranks`` -- Unified attention on a
  ring x Ulysses grid: the regroup, the ring over the regrouped segments, and
  the reverse regroup ("Context parallelism" page, Unified Attention section).

Every function is pinned by the CPU tests in ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force and a library cross-check).
"""
from .attention import attention, attention_rows
from .merge import lse_merge, empty_partial
from .ring import ring_attention
from .permute import ulysses_seq_to_head, ulysses_head_to_seq
from .unified import unified_rank_share, unified_all_ranks
from .permute_any import anything_seq_to_head, anything_head_to_seq, even_split

__all__ = [
    "attention", "attention_rows", "lse_merge", "empty_partial", "ring_attention",
    "ulysses_seq_to_head", "ulysses_head_to_seq", "unified_rank_share", "unified_all_ranks",
    "anything_seq_to_head", "anything_head_to_seq", "even_split",
]
