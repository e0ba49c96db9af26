"""fp64 ring loop: one Q shard against K/V chunks in ring order (test infrastructure only).

"Context parallelism" page, Ring Attention section: each rank attends its
queries to the K/V block it holds, then the block moves on; after N steps every
rank has seen every token.  The "Ring Anything Attention" section pads blocks
to the longest local length for the all-gather and slices each back to its true
length before attention, so only the true lengths ever enter the softmax.  With
K/V resident on one device that is exactly a loop over chunks of the given
lengths, each step producing a partial (output, LSE) that is merged by the
log-sum-exp rule (see ``merge.py``).
"""
from __future__ import annotations

from .attention import attention
from .merge import empty_partial, lse_merge


def ring_attention(q, k, v, chunk_lens, scale=None):
    """q: [..., Sq, d]; k, v: [..., Skv, d] with Skv == sum(chunk_lens).

    Chunk c covers key rows [off_c, off_c + len_c) where off_c is the prefix sum.
    Returns (out, lse) in float64 after merging every chunk in order.
    """
    total = sum(int(n) for n in chunk_lens)
    assert k.shape[-2] == total and v.shape[-2] == total, "chunk lengths must sum to Skv"
    acc_out, acc_lse = empty_partial(q.shape[:-1] + (v.shape[-1],), q.shape[:-1])
    off = 0
    for n in chunk_lens:
        n = int(n)
        assert n >= 0
        blk_out, blk_lse = attention(q, k[..., off:off + n, :], v[..., off:off + n, :], scale=scale)
        acc_out, acc_lse = lse_merge(acc_out, acc_lse, blk_out, blk_lse)
        off += n
    return acc_out, acc_lse
