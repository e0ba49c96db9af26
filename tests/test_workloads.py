"""CPU tests of the seeded workload generator (no method arithmetic lives there)."""
import numpy as np
import pytest
import torch

from context_attention_diffusion_non_amd import workloads as W


def test_bf16_rounding_matches_torch():
    r = np.random.Generator(np.random.PCG64(3))
    x = np.concatenate([r.standard_normal(100_000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, 3.0e38, 1.00390625, 1.01171875],
                                 np.float32)])
    ours = W.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", W.ORDER)
def test_workload_shapes(name):
    wl = W.WORKLOADS[name]
    assert sum(wl.chunk_lens) == wl.S
    assert len(wl.chunk_lens) == wl.ring_degree
    assert wl.q_start + wl.q_len <= wl.S
    assert wl.H % wl.ulysses_degree == 0


def test_sequence_lengths_follow_the_token_counts():
    assert W.WORKLOADS["flux"].S == 512 + 64 * 64
    assert W.WORKLOADS["cogvideox"].S == 226 + 13 * 30 * 45
    assert W.WORKLOADS["mochi"].S == 256 + 28 * 30 * 53
    assert W.WORKLOADS["ring_anything"].chunk_lens == (922, 922, 922, 921, 921)


def test_tiny_inputs_deterministic_and_fp32():
    a = W.make_inputs(W.WORKLOADS["tiny"])
    b = W.make_inputs(W.WORKLOADS["tiny"])
    assert a.q.dtype == np.float32 and a.q_bits is None
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert a.q.shape == (1, 256, 2, 64)


def test_rmsnorm_rows_unit_rms():
    wl = W.WORKLOADS["flux"]
    small = W.Workload(**{**wl.__dict__, "S": 64, "chunk_lens": (32, 32), "q_len": 32})
    x = W.make_inputs(small)
    rms = np.sqrt(np.mean(x.q.astype(np.float64) ** 2, axis=-1))
    assert np.allclose(rms, 1.0, atol=1e-2)           # bf16 rounding leaves ~0.4% wiggle
    assert np.array_equal(W.bf16_bits_to_f32(x.q_bits), x.q)


def test_sample_rows():
    rows = W.sample_rows(11194, seed=9)
    assert rows[0] == 0 and rows[-1] == 11193
    assert np.all(np.diff(rows) > 0)
    assert {127, 128, 255, 256}.issubset(set(rows.tolist()))


def test_random_bhsd_fp16_is_nearest_even_of_the_same_draw():
    x, none = W.random_bhsd(3, (2, 3, 5, 8), "fp32")
    assert none is None
    v, h = W.random_bhsd(3, (2, 3, 5, 8), "fp16")
    assert h.dtype == np.float16 and np.array_equal(v, h.astype(np.float32))
    # nearest representable fp16 of each draw (ties never occur for N(0,1) draws here)
    err = np.abs(v.astype(np.float64) - x.astype(np.float64))
    ulp = np.spacing(np.abs(h)).astype(np.float64)
    assert np.all(err <= 0.5 * ulp)
