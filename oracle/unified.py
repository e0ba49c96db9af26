"""Unified attention, one rank's share and every rank (test infrastructure only).

"Context parallelism" page, Unified Attention section: an all-to-all
redistributes heads and tokens, Ring Attention runs on the result, then the
all-to-all is reversed; the devices form a grid of ulysses_degree x
ring_degree ranks, each in one Ulysses group and one ring group.

Mesh reading (the ParaAttention README example names the mesh dimensions
("ring", "ulysses") with shape (R, U)): rank w = ring_rank * U + ulysses_rank,
row-major.  A rank's Ulysses group is the U ranks sharing its ring_rank, whose
sequence shards are consecutive; its ring group is the R ranks sharing its
ulysses_rank.  Sequence shard w holds tokens [w*S_loc, (w+1)*S_loc).

Layout of q, k, v: the W = R*U sequence shards stacked, ``[W, B, S_loc, H, d]``.

One rank's share (ring_rank, ulysses_rank):
1. Ulysses regroup inside each Ulysses group: group rho's U shards become every
   token of segment rho (U*S_loc tokens) for head group ulysses_rank;
2. ring over the rank's ring group: its query segment against the key/value
   segments of its ring peers in ring order, its own segment first.
The reverse regroup (per Ulysses group) returns outputs by token.
"""
from __future__ import annotations

import numpy as np

from .permute import ulysses_head_to_seq, ulysses_seq_to_head
from .ring import ring_attention


def _group_shards(x, U: int, rho: int):
    return x[rho * U:(rho + 1) * U]


def unified_rank_share(q, k, v, ring_degree: int, ulysses_degree: int, ring_rank: int, ulysses_rank: int,
                       scale=None):
    """(out [B, H/U, U*S_loc, d], lse [B, H/U, U*S_loc]) of one rank, before the reverse regroup."""
    R, U = ring_degree, ulysses_degree
    assert q.shape[0] == R * U and q.shape[3] % U == 0
    qg = ulysses_seq_to_head(_group_shards(q, U, ring_rank), U, ulysses_rank)
    order = [(ring_rank + j) % R for j in range(R)]
    kg = np.concatenate([ulysses_seq_to_head(_group_shards(k, U, rho), U, ulysses_rank) for rho in order], axis=-2)
    vg = np.concatenate([ulysses_seq_to_head(_group_shards(v, U, rho), U, ulysses_rank) for rho in order], axis=-2)
    seg = U * q.shape[2]
    return ring_attention(qg, kg, vg, [seg] * R, scale=scale)


def unified_all_ranks(q, k, v, ring_degree: int, ulysses_degree: int, scale=None):
    """Every rank's share followed by the reverse regroup in each Ulysses group:
    (out [W, B, S_loc, H, d], lse [W, B, S_loc, H]) -- rank w's tokens, all heads."""
    R, U = ring_degree, ulysses_degree
    W, B, S_loc, H, d = q.shape
    out = np.zeros((W, B, S_loc, H, d))
    lse = np.zeros((W, B, S_loc, H))
    for rho in range(R):
        shares = [unified_rank_share(q, k, v, R, U, rho, u, scale=scale) for u in range(U)]
        o = np.stack([s[0] for s in shares], axis=0)              # [U, B, H/U, U*S_loc, d]
        l = np.stack([s[1] for s in shares], axis=0)[..., None]   # [U, B, H/U, U*S_loc, 1]
        out[rho * U:(rho + 1) * U] = ulysses_head_to_seq(o, U, -1)
        lse[rho * U:(rho + 1) * U] = ulysses_head_to_seq(l, U, -1)[..., 0]
    return out, lse
