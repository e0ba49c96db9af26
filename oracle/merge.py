"""fp64 log-sum-exp merge of partial attention results (test infrastructure only).

The pages name the merge only through its numerics: ring attention converts
each step's output and LSE to float32 "for numerical stability"
(``convert_to_fp32`` in the ``ContextParallelConfig`` parameters, "Parallelism"
API page).  The algebra is the log-sum-exp identity: if partial A covers key set
K_a and partial B covers a disjoint key set K_b, then over K_a u K_b

    L   = log(exp(L_a) + exp(L_b))
    out = exp(L_a - L) * out_a + exp(L_b - L) * out_b

An empty partial has L = -inf and contributes nothing; merging with it returns
the other side unchanged, and merging two empty partials gives an empty one
(output 0, LSE -inf).
"""
from __future__ import annotations

import numpy as np


def empty_partial(shape_out, shape_lse):
    """The identity of the merge: output 0 and LSE -inf."""
    return np.zeros(shape_out, np.float64), np.full(shape_lse, -np.inf, np.float64)


def lse_merge(acc_out, acc_lse, blk_out, blk_lse):
    """Merge partial (blk_out, blk_lse) into (acc_out, acc_lse).

    acc_out, blk_out: [..., rows, d]; acc_lse, blk_lse: [..., rows].
    Returns the merged (out, lse) in float64; inputs are not modified.
    """
    ao = np.asarray(acc_out, dtype=np.float64)
    al = np.asarray(acc_lse, dtype=np.float64)
    bo = np.asarray(blk_out, dtype=np.float64)
    bl = np.asarray(blk_lse, dtype=np.float64)
    a_empty = np.isneginf(al)
    b_empty = np.isneginf(bl)
    # L = log(exp(La) + exp(Lb)), evaluated around the larger term
    mx = np.maximum(al, bl)
    safe_mx = np.where(np.isneginf(mx), 0.0, mx)
    wa = np.where(a_empty, 0.0, np.exp(np.where(a_empty, 0.0, al - safe_mx)))
    wb = np.where(b_empty, 0.0, np.exp(np.where(b_empty, 0.0, bl - safe_mx)))
    tot = wa + wb
    both = a_empty & b_empty
    tot_safe = np.where(both, 1.0, tot)
    lse = np.where(both, -np.inf, safe_mx + np.log(tot_safe))
    out = (wa[..., None] * ao + wb[..., None] * bo) / tot_safe[..., None]
    out = np.where(both[..., None], 0.0, out)
    return out, lse
