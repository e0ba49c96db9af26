"""CPU tests: the fp64 oracle against closed forms, invariants, brute force and
library routines (nothing here uses a GPU or the HIP library)."""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests import pins

GOLDEN = pins.GOLDEN


@pytest.mark.parametrize("check", pins.ATTENTION_CHECKS, ids=lambda f: f.__name__)
def test_attention_pins(check):
    check(oracle.attention)


@pytest.mark.parametrize("check", pins.MERGE_CHECKS, ids=lambda f: f.__name__)
def test_merge_pins(check):
    check(oracle.lse_merge)


def test_merge_split_equals_whole():
    pins.check_merge_split_equals_whole(oracle.lse_merge, oracle.attention)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=9), min_size=1, max_size=7), st.integers(0, 10_000))
def test_ring_any_chunking_equals_unsplit(chunk_lens, seed):
    """Any chunking -- uneven, length-1, empty chunks -- merges to unsplit attention."""
    pins.check_ring_matches_unsplit(oracle.ring_attention, oracle.attention, chunk_lens, seed=seed)


def test_ring_anything_lengths():
    """The uneven split of the Ring Anything workload (922/922/922/921/921 over 4608)."""
    lens = (922, 922, 922, 921, 921)
    assert sum(lens) == 4608
    pins.check_ring_matches_unsplit(oracle.ring_attention, oracle.attention, lens, seed=7, sq=5, d=16,
                                    lead=(1,))


def test_ring_all_ranks_equal_unsplit():
    pins.check_ring_all_ranks(oracle.ring_attention, oracle.attention)


def test_pages_unified_example_tolerance():
    """The pages' own check (ParaAttention README): each rank's slice of the
    sharded result against unsplit attention sliced to that rank, rtol 1e-5 and
    atol 1e-3 * world_size, at their shape (one head of it, to stay fast)."""
    with open(os.path.join(GOLDEN, "pages_unified_test.json")) as f:
        g = json.load(f)
    ws = 2
    r = np.random.Generator(np.random.PCG64(g["seed"]))
    S, D = g["S_Q"], g["D"]
    q = r.standard_normal((1, S, D))
    k = r.standard_normal((1, g["S_KV"], D))
    v = r.standard_normal((1, g["S_KV"], D))
    ref_o, _ = oracle.attention(q, k, v)
    share = S // ws
    for rank in range(ws):
        qs = q[:, rank * share:(rank + 1) * share]
        o, _ = oracle.ring_attention(qs, k, v, [g["S_KV"] // ws] * ws)
        np.testing.assert_allclose(o, ref_o[:, rank * share:(rank + 1) * share],
                                   rtol=g["rtol"], atol=g["atol_per_world_size"] * ws)


def test_indivisible_shape_fixture():
    """1008x1008 FLUX gives an odd sequence (4481): not divisible by the 4-way ring
    the pages benchmark, which is why plain ring 'failed' there; the uneven
    ring-anything split still covers every token exactly once."""
    with open(os.path.join(GOLDEN, "indivisible_shapes.json")) as f:
        g = json.load(f)
    ws = g["world_size"]
    for c in g["cases"]:
        side = int(c["shape"].split("x")[0])
        assert 512 + (side // 16) ** 2 == c["S"]
        assert (c["S"] % ws == 0) == c["ring_divisible"]
    S = 4481
    lens = [S // ws + (1 if i < S % ws else 0) for i in range(ws)]
    assert sum(lens) == S and max(lens) - min(lens) <= 1
    pins.check_ring_matches_unsplit(oracle.ring_attention, oracle.attention, [n // 64 for n in lens],
                                    seed=11, sq=3, d=8, lead=(1,))


def test_permute_provenance():
    pins.check_permute_provenance(oracle.ulysses_seq_to_head)


def test_permute_roundtrip():
    pins.check_permute_roundtrip(oracle.ulysses_seq_to_head, oracle.ulysses_head_to_seq)


def test_permute_p1_is_transpose():
    pins.check_permute_is_bshd_to_bhsd(oracle.ulysses_seq_to_head)


def test_attention_rows_are_independent():
    r = np.random.Generator(np.random.PCG64(50))
    q = r.standard_normal((2, 40, 8))
    k = r.standard_normal((2, 33, 8))
    v = r.standard_normal((2, 33, 8))
    rows = np.array([0, 5, 39, 17])
    full_o, full_l = oracle.attention(q, k, v)
    o, l = oracle.attention_rows(q, k, v, rows)
    assert np.array_equal(o, full_o[:, rows]) and np.array_equal(l, full_l[:, rows])


@pytest.mark.parametrize("R,U", [(1, 2), (2, 1), (2, 2), (2, 3), (3, 2), (1, 1)])
def test_unified_equals_unsplit(R, U):
    pins.check_unified_equals_unsplit(oracle.unified_all_ranks, R, U)


def test_unified_share_rows_brute_force():
    pins.check_unified_share_rows(oracle.unified_rank_share)


def test_anything_provenance():
    pins.check_anything_provenance(oracle.anything_seq_to_head)
    pins.check_anything_provenance(oracle.anything_seq_to_head, seq_lens=(2241, 2240), head_lens=(12, 12), B=1, d=1)


def test_anything_roundtrip():
    pins.check_anything_roundtrip(oracle.anything_seq_to_head, oracle.anything_head_to_seq)


def test_anything_even_is_ulysses():
    pins.check_anything_even_is_ulysses(oracle.anything_seq_to_head, oracle.ulysses_seq_to_head)


def test_anything_attention_equals_unsplit():
    pins.check_anything_attention_equals_unsplit(oracle.anything_seq_to_head, oracle.anything_head_to_seq,
                                                 oracle.attention)


def test_even_split_rule():
    assert oracle.even_split(4481, 2) == [2241, 2240]
    assert oracle.even_split(4608, 5) == [922, 922, 922, 921, 921]
    assert oracle.even_split(24, 5) == [5, 5, 5, 5, 4]
    assert sum(oracle.even_split(17, 17)) == 17 and oracle.even_split(3, 5) == [1, 1, 1, 0, 0]
