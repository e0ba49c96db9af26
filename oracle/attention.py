"""Plain fp64 softmax attention with an explicit log-sum-exp (test infrastructure only).

Definition followed: the ``scaled_dot_product_attention(q, k, v,
attn_mask=None, dropout_p=0.0, is_causal=False)`` call of the ParaAttention
README ("Run Unified Attention ... with torch.compile"): no mask, no dropout,
non-causal, default scale 1/sqrt(d).  The LSE is the natural log of the sum of
exp of the *scaled* scores, which is the quantity the ring merge rescales by
(``convert_to_fp32`` in the ``ContextParallelConfig`` parameters).
"""
from __future__ import annotations

import math

import numpy as np


def _plane(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """One (batch, head) plane: q [Sq, d], k [Skv, d], v [Skv, dv] in float64."""
    sq = q.shape[0]
    if k.shape[0] == 0:
        # no keys: nothing to attend to; output 0 and LSE = log(0) = -inf
        return np.zeros((sq, v.shape[1]), np.float64), np.full((sq,), -np.inf, np.float64)
    s = (q @ k.T) * scale                      # scores [Sq, Skv]
    m = np.max(s, axis=1, keepdims=True)       # row max, for a safe exp
    p = np.exp(s - m)                          # unnormalised probabilities
    l = np.sum(p, axis=1, keepdims=True)       # row sums
    o = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention(q, k, v, scale=None):
    """softmax(q k^T * scale) v and its LSE.

    q: [..., Sq, d], k: [..., Skv, d], v: [..., Skv, dv]; leading dims must match.
    Returns (out [..., Sq, dv] float64, lse [..., Sq] float64).
    ``scale=None`` means 1/sqrt(d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lead = q.shape[:-2]
    assert k.shape[:-2] == lead and v.shape[:-2] == lead, "leading dims differ"
    assert k.shape[-2] == v.shape[-2], "k and v lengths differ"
    n = int(np.prod(lead, dtype=np.int64))
    qf = q.reshape((n,) + q.shape[-2:])
    kf = k.reshape((n,) + k.shape[-2:])
    vf = v.reshape((n,) + v.shape[-2:])
    out = np.empty(qf.shape[:-1] + (v.shape[-1],), np.float64)
    lse = np.empty(qf.shape[:-1], np.float64)
    for i in range(qf.shape[0]):
        out[i], lse[i] = _plane(qf[i], kf[i], vf[i], float(scale))
    return out.reshape(lead + out.shape[-2:]), lse.reshape(lead + lse.shape[-1:])


def attention_rows(q, k, v, rows, scale=None):
    """Attention for a subset of query rows only (rows are independent).

    Same as ``attention(q[..., rows, :], k, v)``; used where the full share is
    too large for the CPU.
    """
    q = np.asarray(q)
    return attention(q[..., rows, :], k, v, scale=scale)
