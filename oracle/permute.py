"""Ulysses sequence<->head regroup as a plain numpy transpose (test infrastructure only).

"Context parallelism" page, Ulysses Attention section: after the first
all-to-all a rank holds the whole sequence for its share of the heads; after
attention a second all-to-all hands the results back by token.  The
page requires S and H to divide evenly by the degree P.

Layouts (all row-major):

* sequence-sharded input ``x``: ``[P, B, S_loc, H, d]`` -- shard r holds tokens
  [r*S_loc, (r+1)*S_loc) for all H heads, as rank r holds them;
* head-sharded output for head group g: ``[B, H/P, P*S_loc, d]``, every token
  for heads [g*H/P, (g+1)*H/P).

    out[b, h', r*S_loc + s, e] = x[r, b, s, g*H/P + h', e]

``group=-1`` returns every group stacked: ``[P, B, H/P, S, d]``.
The inverse writes a head-sharded tensor back into the sequence-sharded layout.
"""
from __future__ import annotations

import numpy as np


def ulysses_seq_to_head(x, degree: int, group: int):
    x = np.asarray(x)
    P, B, S_loc, H, d = x.shape
    assert P == degree and H % degree == 0
    hp = H // degree
    groups = range(degree) if group == -1 else [group]
    outs = []
    for g in groups:
        sel = x[:, :, :, g * hp:(g + 1) * hp, :]              # [P, B, S_loc, hp, d]
        t = np.transpose(sel, (1, 3, 0, 2, 4))                 # [B, hp, P, S_loc, d]
        outs.append(np.ascontiguousarray(t).reshape(B, hp, P * S_loc, d))
    return outs[0] if group != -1 else np.stack(outs, axis=0)


def ulysses_head_to_seq(y, degree: int, group: int, base=None):
    """Inverse regroup.

    y: ``[B, H/P, S, d]`` for one group, or ``[P, B, H/P, S, d]`` when group == -1.
    base: the ``[P, B, S/P, H, d]`` tensor to write into (copied, not modified);
    heads outside the written group(s) keep base's values.  If base is None a
    zero tensor is used.
    """
    y = np.asarray(y)
    if group == -1:
        G, B, hp, S, d = y.shape
        assert G == degree
        ys = [y[g] for g in range(degree)]
        groups = list(range(degree))
    else:
        B, hp, S, d = y.shape
        ys = [y]
        groups = [group]
    assert S % degree == 0
    S_loc = S // degree
    H = hp * degree
    out = np.zeros((degree, B, S_loc, H, d), y.dtype) if base is None else np.array(base, copy=True)
    for g, yg in zip(groups, ys):
        t = yg.reshape(B, hp, degree, S_loc, d)                # [B, hp, P, S_loc, d]
        out[:, :, :, g * hp:(g + 1) * hp, :] = np.transpose(t, (2, 0, 3, 1, 4))
    return out
