"""Checks that pin the fp64 oracle to facts outside itself.

Each ``check_*`` takes the function under test as an argument and raises
AssertionError when it disagrees with a closed form, an invariant, a
brute-force evaluation or a library routine.  ``test_oracle_pins.py`` runs them
on the oracle; ``test_oracle_mutants.py`` runs them on deliberately broken
copies of it to show that each plausible mistake is caught by at least one.

Sources of the facts: the attention being computed is the unmasked,
non-causal, dropout-free ``scaled_dot_product_attention`` of the ParaAttention
README ("Run Unified Attention ... with torch.compile"), whose default scale is
1/sqrt(d); the merge is the log-sum-exp identity behind ``convert_to_fp32``
("Parallelism" API page, ``ContextParallelConfig``); the ring loop and its
uneven "anything" split come from the "Context parallelism" page (Ring
Attention, Ring Anything Attention); the permute from its Ulysses Attention
section.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def check_single_key(attn):
    """One key: softmax weight 1, so out == v exactly and lse == the scaled score."""
    r = _rng(1)
    d = 16
    q = r.standard_normal((3, d))
    k = r.standard_normal((1, d))
    v = r.standard_normal((1, 5))
    out, lse = attn(q, k, v)
    assert np.array_equal(out, np.repeat(v, 3, axis=0)), "single key must return v exactly"
    s = np.array([math.fsum(q[i, j] * k[0, j] for j in range(d)) / math.sqrt(d) for i in range(3)])
    assert np.allclose(lse, s, rtol=0, atol=1e-13), "single key lse must equal the scaled score"


def check_zero_query(attn):
    """q == 0: all scores 0, uniform weights: out == column mean of v, lse == ln(Skv)."""
    r = _rng(2)
    skv, d = 37, 8
    q = np.zeros((4, d))
    k = r.standard_normal((skv, d)) * 3.0
    v = r.standard_normal((skv, 6))
    out, lse = attn(q, k, v)
    mean = np.array([math.fsum(v[:, e]) / skv for e in range(6)])
    assert np.allclose(out, mean[None, :], rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(skv), rtol=0, atol=1e-14)


def check_two_keys(attn):
    """Two keys: weights are sigma(s1 - s2) and sigma(s2 - s1); lse = log(e^s1 + e^s2)."""
    r = _rng(3)
    d = 4
    q = r.standard_normal((6, d))
    k = r.standard_normal((2, d))
    v = r.standard_normal((2, 3))
    out, lse = attn(q, k, v)
    for i in range(6):
        s1 = math.fsum(q[i, j] * k[0, j] for j in range(d)) / 2.0
        s2 = math.fsum(q[i, j] * k[1, j] for j in range(d)) / 2.0
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        ref = w1 * v[0] + w2 * v[1]
        assert np.allclose(out[i], ref, rtol=0, atol=1e-14)
        big = max(s1, s2)
        assert abs(lse[i] - (big + math.log(math.exp(s1 - big) + math.exp(s2 - big)))) < 1e-14


def check_large_scores(attn):
    """Scores near 1e3 must not overflow: the result is still the sigmoid closed form."""
    d = 4
    q = np.array([[40.0, 0.0, 0.0, 0.0]])
    k = np.array([[50.0, 0.0, 0.0, 0.0], [49.9, 0.0, 0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    out, lse = attn(q, k, v)
    s1, s2 = 40 * 50 / 2.0, 40 * 49.9 / 2.0
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert np.allclose(out[0], [w1, 1.0 - w1], rtol=0, atol=1e-12)
    assert abs(lse[0] - (s1 + math.log1p(math.exp(s2 - s1)))) < 1e-9


def _brute(q, k, v, scale):
    """Pure-Python attention on tiny inputs, exact sums via math.fsum, no max shift."""
    sq, d = q.shape
    skv = k.shape[0]
    outs, lses = [], []
    for i in range(sq):
        s = [math.fsum(q[i, t] * k[j, t] for t in range(d)) * scale for j in range(skv)]
        e = [math.exp(x) for x in s]
        z = math.fsum(e)
        outs.append([math.fsum(e[j] * v[j, c] for j in range(skv)) / z for c in range(v.shape[1])])
        lses.append(math.log(z))
    return np.array(outs), np.array(lses)


def check_brute_force(attn):
    """Tiny random cases against the pure-Python definition (lse without max shift)."""
    for seed, (sq, skv, d) in enumerate([(3, 5, 4), (7, 2, 8), (1, 9, 3), (5, 5, 5)]):
        r = _rng(100 + seed)
        q = r.standard_normal((sq, d))
        k = r.standard_normal((skv, d))
        v = r.standard_normal((skv, 3))
        out, lse = attn(q, k, v)
        bo, bl = _brute(q, k, v, 1.0 / math.sqrt(d))
        assert np.allclose(out, bo, rtol=0, atol=1e-13), f"out differs from brute force (seed {seed})"
        assert np.allclose(lse, bl, rtol=0, atol=1e-13), f"lse differs from brute force (seed {seed})"


def check_explicit_scale(attn):
    """An explicit scale replaces 1/sqrt(d)."""
    r = _rng(5)
    q = r.standard_normal((4, 6))
    k = r.standard_normal((7, 6))
    v = r.standard_normal((7, 2))
    out, lse = attn(q, k, v, scale=0.3)
    bo, bl = _brute(q, k, v, 0.3)
    assert np.allclose(out, bo, atol=1e-13) and np.allclose(lse, bl, atol=1e-13)


def check_invariances(attn):
    """Joint K/V row permutation: unchanged.  Key shift by u: out unchanged,
    lse shifts by scale*q.u.  Linearity in v."""
    r = _rng(6)
    sq, skv, d = 9, 31, 16
    q = r.standard_normal((sq, d))
    k = r.standard_normal((skv, d))
    v = r.standard_normal((skv, 5))
    out, lse = attn(q, k, v)
    perm = r.permutation(skv)
    o2, l2 = attn(q, k[perm], v[perm])
    assert np.allclose(o2, out, atol=1e-13) and np.allclose(l2, lse, atol=1e-13)
    u = r.standard_normal(d)
    o3, l3 = attn(q, k + u[None, :], v)
    assert np.allclose(o3, out, atol=1e-12)
    assert np.allclose(l3, lse + (q @ u) / math.sqrt(d), atol=1e-12)
    v2 = r.standard_normal((skv, 5))
    o4, _ = attn(q, k, 2.0 * v - 3.0 * v2)
    o5, _ = attn(q, k, v2)
    assert np.allclose(o4, 2.0 * out - 3.0 * o5, atol=1e-12)


def check_batched_planes(attn):
    """Leading (batch, head) dims are independent planes."""
    r = _rng(7)
    q = r.standard_normal((2, 3, 5, 8))
    k = r.standard_normal((2, 3, 6, 8))
    v = r.standard_normal((2, 3, 6, 8))
    out, lse = attn(q, k, v)
    for b in range(2):
        for h in range(3):
            o, l = attn(q[b, h], k[b, h], v[b, h])
            assert np.array_equal(o, out[b, h]) and np.array_equal(l, lse[b, h])


def check_no_keys(attn):
    """Zero keys: output 0, lse -inf (log of an empty sum)."""
    q = np.ones((3, 4))
    out, lse = attn(q, np.zeros((0, 4)), np.zeros((0, 2)))
    assert out.shape == (3, 2) and np.all(out == 0.0) and np.all(np.isneginf(lse))


def check_torch_sdpa(attn):
    """Library cross-check: torch's CPU SDPA and logsumexp in float64."""
    import torch
    r = _rng(8)
    q = r.standard_normal((2, 3, 17, 32))
    k = r.standard_normal((2, 3, 23, 32))
    v = r.standard_normal((2, 3, 23, 32))
    out, lse = attn(q, k, v)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=None, dropout_p=0.0,
                                                           is_causal=False)
    ref_lse = torch.logsumexp(tq @ tk.transpose(-1, -2) / math.sqrt(32), dim=-1)
    assert np.allclose(out, ref.numpy(), atol=1e-12)
    assert np.allclose(lse, ref_lse.numpy(), atol=1e-12)


ATTENTION_CHECKS = [check_single_key, check_zero_query, check_two_keys, check_large_scores,
                    check_brute_force, check_explicit_scale, check_invariances, check_batched_planes,
                    check_no_keys, check_torch_sdpa]


# --------------------------------------------------------------------------
# merge
# --------------------------------------------------------------------------

def check_merge_identity(merge):
    """Merging with an empty partial (lse -inf) returns the other side exactly."""
    r = _rng(20)
    o = r.standard_normal((4, 8))
    l = r.standard_normal(4)
    e_o, e_l = np.zeros((4, 8)), np.full(4, -np.inf)
    mo, ml = merge(o, l, e_o, e_l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = merge(e_o, e_l, o, l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = merge(e_o, e_l, e_o, e_l)
    assert np.all(mo == 0.0) and np.all(np.isneginf(ml))


def check_merge_self(merge):
    """A partial merged with an identical one: same output, lse + ln 2."""
    r = _rng(21)
    o = r.standard_normal((5, 3))
    l = r.standard_normal(5) * 10
    mo, ml = merge(o, l, o, l)
    assert np.allclose(mo, o, atol=1e-14) and np.allclose(ml, l + math.log(2.0), atol=1e-13)


def check_merge_closed_form(merge):
    """Two scalar partials: weights e^La/(e^La+e^Lb); computed with fsum in pure Python."""
    for la, lb, oa, ob in [(0.0, 0.0, 1.0, 3.0), (2.0, -1.0, 5.0, -7.0), (-3.5, 4.25, 0.5, 0.25),
                           (700.0, 699.0, 1.0, 2.0)]:
        mo, ml = merge(np.array([[oa]]), np.array([la]), np.array([[ob]]), np.array([lb]))
        big = max(la, lb)
        ea, eb = math.exp(la - big), math.exp(lb - big)
        assert abs(ml[0] - (big + math.log(ea + eb))) < 1e-12
        assert abs(mo[0, 0] - (ea * oa + eb * ob) / (ea + eb)) < 1e-12


def check_merge_commutes(merge):
    r = _rng(22)
    a_o, b_o = r.standard_normal((6, 4)), r.standard_normal((6, 4))
    a_l, b_l = r.standard_normal(6) * 5, r.standard_normal(6) * 5
    x = merge(a_o, a_l, b_o, b_l)
    y = merge(b_o, b_l, a_o, a_l)
    assert np.allclose(x[0], y[0], atol=1e-14) and np.allclose(x[1], y[1], atol=1e-14)


def check_merge_split_equals_whole(merge, attn):
    """Attention over two disjoint key sets, merged, equals attention over their union."""
    r = _rng(23)
    q = r.standard_normal((7, 8))
    k = r.standard_normal((19, 8))
    v = r.standard_normal((19, 4))
    whole = attn(q, k, v)
    a = attn(q, k[:6], v[:6])
    b = attn(q, k[6:], v[6:])
    m = merge(a[0], a[1], b[0], b[1])
    assert np.allclose(m[0], whole[0], atol=1e-13) and np.allclose(m[1], whole[1], atol=1e-13)


MERGE_CHECKS = [check_merge_identity, check_merge_self, check_merge_closed_form, check_merge_commutes]


# --------------------------------------------------------------------------
# ring
# --------------------------------------------------------------------------

def check_ring_matches_unsplit(ring, attn, chunk_lens, seed=30, sq=11, d=8, lead=(2,)):
    r = _rng(seed)
    skv = sum(chunk_lens)
    q = r.standard_normal(lead + (sq, d))
    k = r.standard_normal(lead + (skv, d))
    v = r.standard_normal(lead + (skv, d))
    ro, rl = ring(q, k, v, chunk_lens)
    if skv == 0:
        assert np.all(ro == 0) and np.all(np.isneginf(rl))
        return
    uo, ul = attn(q, k, v)
    assert np.allclose(ro, uo, rtol=0, atol=1e-12)
    assert np.allclose(rl, ul, rtol=0, atol=1e-12)


def check_ring_all_ranks(ring, attn, S=48, P=4, d=8):
    """Every rank of a ring, simulated: rank r's Q rows against all chunks; the
    concatenation over ranks equals unsplit attention ("after one full loop,
    every GPU has seen every token's K/V")."""
    r = _rng(31)
    q = r.standard_normal((3, S, d))
    k = r.standard_normal((3, S, d))
    v = r.standard_normal((3, S, d))
    lens = [S // P] * P
    parts = []
    for rank in range(P):
        qs = q[:, rank * (S // P):(rank + 1) * (S // P)]
        # rank r sees its own chunk first, then r+1, ...; the order must not matter
        order = [(rank + i) % P for i in range(P)]
        kk = np.concatenate([k[:, c * (S // P):(c + 1) * (S // P)] for c in order], axis=1)
        vv = np.concatenate([v[:, c * (S // P):(c + 1) * (S // P)] for c in order], axis=1)
        parts.append(ring(qs, kk, vv, lens))
    cat_o = np.concatenate([p[0] for p in parts], axis=1)
    cat_l = np.concatenate([p[1] for p in parts], axis=1)
    uo, ul = attn(q, k, v)
    # the pages' own tolerance for sharded vs unsplit (ParaAttention README test):
    # rtol 1e-5, atol 1e-3 * world_size; the fp64 oracle is far inside it
    assert np.allclose(cat_o, uo, rtol=1e-5, atol=1e-3 * P)
    assert np.allclose(cat_o, uo, rtol=0, atol=1e-12) and np.allclose(cat_l, ul, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# permute
# --------------------------------------------------------------------------

def _encoded_shards(P, B, S_loc, H, d):
    """Each element's value encodes where it sits: (rank, b, s, h, e) -> unique int."""
    r, b, s, h, e = np.meshgrid(np.arange(P), np.arange(B), np.arange(S_loc), np.arange(H), np.arange(d),
                                indexing="ij")
    return ((((r * B + b) * S_loc + s) * H + h) * d + e).astype(np.int64)


def _decode(val, P, B, S_loc, H, d):
    e = val % d
    val //= d
    h = val % H
    val //= H
    s = val % S_loc
    val //= S_loc
    b = val % B
    r = val // B
    return r, b, s, h, e


def check_permute_provenance(seq_to_head):
    """Every element of the head-sharded output came from exactly the right place:
    token t = r*S_loc + s of head g*H/P + h' (pure-Python loops over a tiny case)."""
    P, B, S_loc, H, d = 3, 2, 4, 6, 5
    x = _encoded_shards(P, B, S_loc, H, d)
    hp = H // P
    for g in range(P):
        out = seq_to_head(x, P, g)
        assert out.shape == (B, hp, P * S_loc, d)
        for b in range(B):
            for hh in range(hp):
                for t in range(P * S_loc):
                    for e in range(d):
                        rr, bb, ss, h_src, ee = _decode(int(out[b, hh, t, e]), P, B, S_loc, H, d)
                        assert (rr, bb, ss, h_src, ee) == (t // S_loc, b, t % S_loc, g * hp + hh, e)
    allg = seq_to_head(x, P, -1)
    for g in range(P):
        assert np.array_equal(allg[g], seq_to_head(x, P, g))


def check_permute_roundtrip(seq_to_head, head_to_seq):
    P, B, S_loc, H, d = 2, 1, 5, 4, 3
    x = _encoded_shards(P, B, S_loc, H, d)
    back = head_to_seq(seq_to_head(x, P, -1), P, -1)
    assert np.array_equal(back, x)
    # one group written back leaves the other group's heads as they were in base
    base = np.full_like(x, -1)
    one = head_to_seq(seq_to_head(x, P, 1), P, 1, base=base)
    assert np.array_equal(one[:, :, :, 2:4, :], x[:, :, :, 2:4, :])
    assert np.all(one[:, :, :, 0:2, :] == -1)


def check_permute_is_bshd_to_bhsd(seq_to_head):
    """With P = 1 the regroup is the plain [B,S,H,d] -> [B,H,S,d] transpose."""
    r = _rng(40)
    x = r.standard_normal((1, 2, 7, 3, 4))
    out = seq_to_head(x, 1, 0)
    for b in range(2):
        for h in range(3):
            for s in range(7):
                assert np.array_equal(out[b, h, s], x[0, b, s, h])


# --------------------------------------------------------------------------
# unified (Ulysses x Ring)
# --------------------------------------------------------------------------

def _torch_sdpa_bshd(q, k, v):
    """Unsplit attention of full-sequence [B, S, H, d] tensors by torch's CPU SDPA in
    float64 (a library routine), returned as [B, S, H, d] and the LSE [B, S, H]."""
    import torch
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()
    d = q.shape[-1]
    lse = torch.logsumexp(qt @ kt.transpose(-1, -2) / math.sqrt(d), dim=-1).numpy()
    return np.transpose(out, (0, 2, 1, 3)), np.transpose(lse, (0, 2, 1))


def check_unified_equals_unsplit(unified_all, R, U, seed=50, B=2, S_loc=3, H_per=2, d=4):
    """Every rank's share on a ring_degree x ulysses_degree grid, regrouped back by
    token, equals unsplit attention of the whole sequence (torch SDPA, fp64):
    the composition the pages describe loses nothing and reorders nothing."""
    r = _rng(seed + 7 * R + U)
    W, H = R * U, H_per * U
    full = [r.standard_normal((B, W * S_loc, H, d)) for _ in range(3)]
    shards = [np.ascontiguousarray(x.reshape(B, W, S_loc, H, d).transpose(1, 0, 2, 3, 4)) for x in full]
    out, lse = unified_all(*shards, R, U)
    ref_out, ref_lse = _torch_sdpa_bshd(*full)
    ref_out = ref_out.reshape(B, W, S_loc, H, d).transpose(1, 0, 2, 3, 4)
    ref_lse = ref_lse.reshape(B, W, S_loc, H).transpose(1, 0, 2, 3)
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    assert np.abs(out - ref_out).max() < 1e-12, f"unified {R}x{U} differs from unsplit attention"
    assert np.abs(lse - ref_lse).max() < 1e-12, f"unified {R}x{U} lse differs from unsplit"


def check_unified_share_rows(unified_share, R=2, U=2, seed=60, B=1, S_loc=2, H_per=1, d=4):
    """One rank's share before the reverse regroup is attention of ITS Ulysses
    group's tokens (segment ring_rank) for ITS head group against every token:
    row by row against a pure-Python brute force."""
    r = _rng(seed)
    W, H = R * U, H_per * U
    full = [r.standard_normal((B, W * S_loc, H, d)) for _ in range(3)]
    shards = [np.ascontiguousarray(x.reshape(B, W, S_loc, H, d).transpose(1, 0, 2, 3, 4)) for x in full]
    q, k, v = full
    S = W * S_loc
    for rho in range(R):
        for u in range(U):
            out, lse = unified_share(*shards, R, U, rho, u)
            assert out.shape == (B, H_per, U * S_loc, d)
            for b in range(B):
                for hh in range(H_per):
                    h = u * H_per + hh
                    for i in range(U * S_loc):
                        t = rho * U * S_loc + i
                        sc = [math.fsum(q[b, t, h, e] * k[b, j, h, e] for e in range(d)) / math.sqrt(d)
                              for j in range(S)]
                        m = max(sc)
                        w = [math.exp(s - m) for s in sc]
                        z = math.fsum(w)
                        for e in range(d):
                            ref = math.fsum(w[j] * v[b, j, h, e] for j in range(S)) / z
                            assert abs(out[b, hh, i, e] - ref) < 1e-12
                        assert abs(lse[b, hh, i] - (m + math.log(z))) < 1e-12


# --------------------------------------------------------------------------
# Ulysses Anything (uneven shards and head groups)
# --------------------------------------------------------------------------

def _encoded_uneven(seq_lens, B, H, d):
    """Shards whose values encode (token t, b, head h, e) of the whole sequence."""
    S = sum(seq_lens)
    t, b, h, e = np.meshgrid(np.arange(S), np.arange(B), np.arange(H), np.arange(d), indexing="ij")
    full = (((t * B + b) * H + h) * d + e).astype(np.int64)       # [S, B, H, d]
    full = np.transpose(full, (1, 0, 2, 3))                          # [B, S, H, d]
    off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
    return [np.ascontiguousarray(full[:, off[r]:off[r + 1]]) for r in range(len(seq_lens))]


def check_anything_provenance(seq_to_head, seq_lens=(5, 4, 4), head_lens=(3, 2, 2), B=2, d=3):
    """Every element of head group g came from token t, head hoff_g + h' of the
    whole sequence (pure-Python loops, uneven tokens and heads)."""
    H = sum(head_lens)
    S = sum(seq_lens)
    shards = _encoded_uneven(list(seq_lens), B, H, d)
    hoff = np.concatenate([[0], np.cumsum(head_lens)]).astype(int)
    for g in range(len(head_lens)):
        out = seq_to_head(shards, list(head_lens), g)
        assert out.shape == (B, head_lens[g], S, d)
        for b in range(B):
            for hh in range(head_lens[g]):
                for t in range(S):
                    for e in range(d):
                        val = int(out[b, hh, t, e])
                        assert val == (((t * B + b) * H + hoff[g] + hh) * d + e)


def check_anything_roundtrip(seq_to_head, head_to_seq, seq_lens=(7, 6, 6, 6), head_lens=(2, 2, 1, 1), B=1, d=4):
    H = sum(head_lens)
    shards = _encoded_uneven(list(seq_lens), B, H, d)
    groups = [seq_to_head(shards, list(head_lens), g) for g in range(len(head_lens))]
    back = head_to_seq(groups, list(seq_lens))
    for r in range(len(seq_lens)):
        assert np.array_equal(back[r], shards[r])


def check_anything_even_is_ulysses(seq_to_head, ulysses):
    """Even lengths: the Anything regroup equals the plain Ulysses one."""
    r = _rng(70)
    P, B, S_loc, H, d = 3, 2, 4, 6, 5
    x = r.standard_normal((P, B, S_loc, H, d))
    for g in range(P):
        assert np.array_equal(seq_to_head([x[i] for i in range(P)], [H // P] * P, g), ulysses(x, P, g))


def check_anything_attention_equals_unsplit(seq_to_head, head_to_seq, attn, seq_lens=(5, 4, 4), head_lens=(2, 1, 1)):
    """Regroup, attention per head group over the whole sequence, reverse regroup:
    every rank's tokens get unsplit attention (torch SDPA, fp64)."""
    r = _rng(71)
    B, d = 2, 4
    H, S = sum(head_lens), sum(seq_lens)
    full = [r.standard_normal((B, S, H, d)) for _ in range(3)]
    off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
    shards = [[np.ascontiguousarray(x[:, off[i]:off[i + 1]]) for i in range(len(seq_lens))] for x in full]
    outs = []
    for g in range(len(head_lens)):
        qg, kg, vg = (seq_to_head(s, list(head_lens), g) for s in shards)
        outs.append(attn(qg, kg, vg)[0])
    back = head_to_seq(outs, list(seq_lens))
    ref, _ = _torch_sdpa_bshd(*full)
    for i in range(len(seq_lens)):
        assert np.abs(back[i] - ref[:, off[i]:off[i + 1]]).max() < 1e-12
