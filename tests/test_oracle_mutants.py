"""CPU tests: plausible mistakes planted in copies of the oracle must each fail
at least one pin.  The mutants live here, on the CPU; the oracle itself is
untouched."""
import math

import numpy as np
import pytest

import oracle
from tests import pins


def _attn_from(plane_fn):
    def attn(q, k, v, scale=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        d = q.shape[-1]
        sc = 1.0 / math.sqrt(d) if scale is None else scale
        lead = q.shape[:-2]
        n = int(np.prod(lead, dtype=np.int64))
        qf, kf, vf = (x.reshape((n,) + x.shape[-2:]) for x in (q, k, v))
        outs, lses = [], []
        for i in range(qf.shape[0]):
            if kf[i].shape[0] == 0:
                outs.append(np.zeros((qf[i].shape[0], vf[i].shape[1])))
                lses.append(np.full(qf[i].shape[0], -np.inf))
                continue
            o, l = plane_fn(qf[i], kf[i], vf[i], sc, d)
            outs.append(o)
            lses.append(l)
        out = np.stack(outs).reshape(lead + outs[0].shape)
        lse = np.stack(lses).reshape(lead + lses[0].shape)
        return out, lse
    return attn


def _softmax_parts(s):
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return m, p, p.sum(axis=1, keepdims=True)


def m_no_scale(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def m_scale_1_over_d(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T * (sc * sc if sc != 1.0 / math.sqrt(d) else 1.0 / d))
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def m_no_max_shift(q, k, v, sc, d):
    s = q @ k.T * sc
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(s)
        l = p.sum(axis=1, keepdims=True)
        return (p @ v) / l, np.log(l[:, 0])


def m_lse_drops_max(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T * sc)
    return (p @ v) / l, np.log(l[:, 0])


def m_lse_log2(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T * sc)
    return (p @ v) / l, m[:, 0] + np.log2(l[:, 0])


def m_divide_by_count(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T * sc)
    return (p @ v) / k.shape[0], m[:, 0] + np.log(l[:, 0])


def m_sign_flip(q, k, v, sc, d):
    s = q @ k.T * sc
    m = s.min(axis=1, keepdims=True)
    p = np.exp(m - s)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, -m[:, 0] + np.log(l[:, 0])


def m_softmax_wrong_axis(q, k, v, sc, d):
    s = q @ k.T * sc
    m = s.max(axis=0, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=0, keepdims=True)
    pn = p / l
    return pn @ v, np.log(np.exp(s).sum(axis=1))


def m_transposed_k(q, k, v, sc, d):
    # uses k's columns as keys where shapes allow (square blocks), else falls back
    kk = k.T if k.shape[0] == k.shape[1] else k[::-1]
    m, p, l = _softmax_parts(q @ kk.T * sc)
    return (p @ v) / l, m[:, 0] + np.log(l[:, 0])


def m_values_reversed(q, k, v, sc, d):
    m, p, l = _softmax_parts(q @ k.T * sc)
    return (p @ v[::-1]) / l, m[:, 0] + np.log(l[:, 0])


ATTN_MUTANTS = [m_no_scale, m_scale_1_over_d, m_no_max_shift, m_lse_drops_max, m_lse_log2,
                m_divide_by_count, m_sign_flip, m_softmax_wrong_axis, m_transposed_k, m_values_reversed]


def _fails_some(checks, *args):
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c(*args)
        except (AssertionError, ValueError, FloatingPointError, ZeroDivisionError, IndexError):
            return True
    return False


@pytest.mark.parametrize("mut", ATTN_MUTANTS, ids=lambda f: f.__name__)
def test_attention_mutant_is_caught(mut):
    assert _fails_some(pins.ATTENTION_CHECKS, _attn_from(mut)), f"{mut.__name__} passed every pin"


def test_unmutated_copy_passes():
    def plane(q, k, v, sc, d):
        m, p, l = _softmax_parts(q @ k.T * sc)
        return (p @ v) / l, m[:, 0] + np.log(l[:, 0])
    for c in pins.ATTENTION_CHECKS:
        c(_attn_from(plane))


def mm_swapped_weights(ao, al, bo, bl):
    o, l = oracle.lse_merge(ao, al, bo, bl)
    mx = np.maximum(al, bl)
    wa = np.exp(bl - mx)
    wb = np.exp(al - mx)
    with np.errstate(all="ignore"):
        return (wa[..., None] * ao + wb[..., None] * bo) / (wa + wb)[..., None], l


def mm_unnormalised(ao, al, bo, bl):
    mx = np.maximum(al, bl)
    with np.errstate(all="ignore"):
        wa, wb = np.exp(al - mx), np.exp(bl - mx)
        return wa[..., None] * ao + wb[..., None] * bo, mx + np.log(wa + wb)


def mm_lse_is_max(ao, al, bo, bl):
    o, _ = oracle.lse_merge(ao, al, bo, bl)
    return o, np.maximum(al, bl)


def mm_average(ao, al, bo, bl):
    return 0.5 * (np.asarray(ao) + np.asarray(bo)), np.logaddexp(al, bl)


MERGE_MUTANTS = [mm_swapped_weights, mm_unnormalised, mm_lse_is_max, mm_average]


@pytest.mark.parametrize("mut", MERGE_MUTANTS, ids=lambda f: f.__name__)
def test_merge_mutant_is_caught(mut):
    caught = _fails_some(pins.MERGE_CHECKS, mut)
    if not caught:
        try:
            pins.check_merge_split_equals_whole(mut, oracle.attention)
        except AssertionError:
            caught = True
    assert caught, f"{mut.__name__} passed every merge pin"


def pm_rank_fastest(x, degree, group):
    P, B, S_loc, H, d = x.shape
    hp = H // degree
    sel = x[:, :, :, group * hp:(group + 1) * hp, :]
    t = np.transpose(sel, (1, 3, 2, 0, 4))          # token order s*P + r instead of r*S_loc + s
    return np.ascontiguousarray(t).reshape(B, hp, P * S_loc, d)


def pm_strided_heads(x, degree, group):
    P, B, S_loc, H, d = x.shape
    hp = H // degree
    sel = x[:, :, :, group::degree, :]              # heads g, g+P, ... instead of a contiguous slice
    t = np.transpose(sel, (1, 3, 0, 2, 4))
    return np.ascontiguousarray(t).reshape(B, hp, P * S_loc, d)


@pytest.mark.parametrize("mut", [pm_rank_fastest, pm_strided_heads], ids=lambda f: f.__name__)
def test_permute_mutant_is_caught(mut):
    def wrapped(x, degree, group):
        if group == -1:
            return np.stack([mut(x, degree, g) for g in range(degree)])
        return mut(x, degree, group)
    with pytest.raises(AssertionError):
        pins.check_permute_provenance(wrapped)


# --- unified: wrong mesh order, ring order not starting at the own segment,
# reverse regroup into the wrong Ulysses group ---

def mu_mesh_transposed(q, k, v, R, U, ring_rank, ulysses_rank, scale=None):
    """Ulysses group taken as every R-th shard (rank = ulysses_rank * R + ring_rank)."""
    W = R * U
    perm = [u * R + rho for rho in range(R) for u in range(U)]
    return oracle.unified_rank_share(q[perm], k[perm], v[perm], R, U, ring_rank, ulysses_rank, scale)


def mu_query_from_group_zero(q, k, v, R, U, ring_rank, ulysses_rank, scale=None):
    """Queries always taken from the first Ulysses group's segment."""
    qq = np.array(q, copy=True)
    qq[ring_rank * U:(ring_rank + 1) * U] = q[0:U]
    return oracle.unified_rank_share(qq, k, v, R, U, ring_rank, ulysses_rank, scale)


def mu_heads_of_next_group(q, k, v, R, U, ring_rank, ulysses_rank, scale=None):
    """Keys and values of the wrong head group."""
    out_q = oracle.unified_rank_share(q, k, v, R, U, ring_rank, ulysses_rank, scale)
    if U == 1:
        return out_q
    kk = np.roll(k, -(k.shape[3] // U), axis=3)
    vv = np.roll(v, -(v.shape[3] // U), axis=3)
    return oracle.unified_rank_share(q, kk, vv, R, U, ring_rank, ulysses_rank, scale)


@pytest.mark.parametrize("mut", [mu_mesh_transposed, mu_query_from_group_zero, mu_heads_of_next_group],
                         ids=lambda f: f.__name__)
def test_unified_mutant_is_caught(mut):
    def all_ranks(q, k, v, R, U):
        W, B, S_loc, H, d = q.shape
        out = np.zeros((W, B, S_loc, H, d))
        lse = np.zeros((W, B, S_loc, H))
        for rho in range(R):
            shares = [mut(q, k, v, R, U, rho, u) for u in range(U)]
            o = np.stack([s[0] for s in shares])
            l = np.stack([s[1] for s in shares])[..., None]
            out[rho * U:(rho + 1) * U] = oracle.ulysses_head_to_seq(o, U, -1)
            lse[rho * U:(rho + 1) * U] = oracle.ulysses_head_to_seq(l, U, -1)[..., 0]
        return out, lse
    caught = False
    for R, U in [(2, 2), (3, 2)]:
        try:
            pins.check_unified_equals_unsplit(all_ranks, R, U)
        except AssertionError:
            caught = True
    try:
        pins.check_unified_share_rows(mut)
    except AssertionError:
        caught = True
    assert caught, f"{mut.__name__} passed every unified pin"


def test_unified_reverse_regroup_mutant_is_caught():
    """Reverse regroup writing each rank's heads into the neighbouring Ulysses group."""
    def all_ranks(q, k, v, R, U):
        out, lse = oracle.unified_all_ranks(q, k, v, R, U)
        return np.roll(out, U, axis=0), np.roll(lse, U, axis=0)
    with pytest.raises(AssertionError):
        pins.check_unified_equals_unsplit(all_ranks, 2, 2)


# --- Ulysses Anything: even-split assumptions planted in a copy of the regroup ---

def ma_even_head_offsets(shards, head_lens, group):
    """Head offset g * (H // P) instead of the prefix sum of the given head counts."""
    H = shards[0].shape[2]
    P = len(shards)
    h0 = group * (H // P)
    full = np.concatenate([np.asarray(x)[:, :, h0:h0 + head_lens[group], :] for x in shards], axis=1)
    return np.ascontiguousarray(np.transpose(full, (0, 2, 1, 3)))


def ma_shards_reversed(shards, head_lens, group):
    """Shards concatenated in reverse rank order."""
    return oracle.anything_seq_to_head(list(reversed(shards)), head_lens, group)


@pytest.mark.parametrize("mut", [ma_even_head_offsets, ma_shards_reversed], ids=lambda f: f.__name__)
def test_anything_mutant_is_caught(mut):
    with pytest.raises(AssertionError):
        pins.check_anything_provenance(mut)
