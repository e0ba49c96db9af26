"""Ulysses Anything regroup: uneven sequence shards and head groups (test infrastructure only).

"Context parallelism" page, Ulysses Anything Attention section: plain Ulysses
needs the sequence length and the head count to divide by ulysses_degree; the
Anything variant removes both requirements (and the tables show it running
FLUX at 1008x1008, S = 4481 tokens, where every even split fails).  The pages
give no split rule; reading: rank r holds ``seq_lens[r]`` consecutive tokens
and, after the regroup, ``head_lens[r]`` consecutive heads, both given
explicitly (the default used by the tests gives the first ``n mod P`` ranks one
more, as ``numpy.array_split`` does).

Layouts (all row-major):

* sequence shards, packed back to back: shard r is ``[B, seq_lens[r], H, d]``;
* head group g: ``[B, head_lens[g], S, d]`` with S = sum(seq_lens):

    out_g[b, h', off_r + s, e] = shard_r[b, s, hoff_g + h', e]

  where off_r and hoff_g are prefix sums of the lengths.
"""
from __future__ import annotations

import numpy as np


def even_split(n: int, parts: int):
    """Lengths of ``parts`` consecutive pieces of n, the first n mod parts one longer."""
    base, extra = divmod(n, parts)
    return [base + (1 if i < extra else 0) for i in range(parts)]


def _offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(int)


def anything_seq_to_head(shards, head_lens, group: int):
    """shards: list of P arrays [B, s_r, H, d].  Returns [B, head_lens[group], S, d]."""
    P = len(shards)
    assert len(head_lens) == P and sum(head_lens) == shards[0].shape[2]
    hoff = _offsets(head_lens)
    h0, h1 = hoff[group], hoff[group + 1]
    # every token of the sequence, in shard order, for the group's heads
    full = np.concatenate([np.asarray(x)[:, :, h0:h1, :] for x in shards], axis=1)   # [B, S, hl, d]
    return np.ascontiguousarray(np.transpose(full, (0, 2, 1, 3)))


def anything_head_to_seq(groups, seq_lens):
    """Inverse: groups = list of P arrays [B, head_lens[g], S, d] -> list of shards [B, s_r, H, d]."""
    full = np.concatenate([np.transpose(np.asarray(y), (0, 2, 1, 3)) for y in groups], axis=2)   # [B, S, H, d]
    off = _offsets(seq_lens)
    return [np.ascontiguousarray(full[:, off[r]:off[r + 1]]) for r in range(len(seq_lens))]
