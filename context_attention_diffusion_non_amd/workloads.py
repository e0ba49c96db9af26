"""Seeded synthetic workloads for per-rank context-parallel attention.

This module only draws inputs and describes shapes. It holds none of the
attention arithmetic, so the fp64 oracle and the HIP path can both be fed from
it without sharing any of the method.

The five workloads are rank shares of the sequence lengths the pages run:

* a tiny ring share (fp32, parity only);
* FLUX.1-dev at 1024x1024: 512 text + 4096 image tokens, 24 heads, d=128
  ("Context parallelism", Ring Attention section, FLUX.1-dev example; the
  ParaAttention README "Usage" FLUX example);
* CogVideoX-5b: 226 text + 13x30x45 video tokens, 48 heads, d=64, Ulysses
  degree 2 (the ParaAttention README lists CogVideoX among its examples);
* Mochi-1-preview: 256 text + 28x30x53 video tokens, 24 heads, d=128, ring
  degree 4 (ParaAttention README, "Run Mochi with Parallel Inference");
* Ring Anything with an uneven 5-way split and a CFG batch of 2
  ("Context parallelism", Ring Anything Attention section).

Recipe: one ``numpy.random.Generator(PCG64(seed))`` per workload; draw q, then
k, then v, each full sequence, token-major ``[B, S, H, d]`` float32 N(0, 1).
Where the workload says so, q and k are RMS-normalised per (b, token, head)
row with unit weight and eps 1e-6.  Then everything except the fp32 tiny case
is rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

RMS_EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    d: int
    dtype: str                      # "bf16" or "fp32": the dtype handed to the library
    rmsnorm_qk: bool
    ring_degree: int
    chunk_lens: Tuple[int, ...]     # K/V chunk lengths in ring order (sum == S)
    q_start: int                    # first query row of the rank-0 share
    q_len: int                      # query rows in the share
    seed: int
    ulysses_degree: int = 1         # >1: inputs arrive as seq-shards and are permuted to heads
    ulysses_group: int = 0          # head group this rank keeps after the permute
    note: str = ""

    @property
    def heads_local(self) -> int:
        return self.H // self.ulysses_degree

    @property
    def flops(self) -> float:
        """Algorithmic attention flops of the share: 4 * B * H_local * Sq * Skv * d."""
        return 4.0 * self.B * self.heads_local * self.q_len * self.S * self.d


def _even(S: int, n: int) -> Tuple[int, ...]:
    assert S % n == 0
    return tuple([S // n] * n)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", B=1, H=2, S=256, d=64, dtype="fp32", rmsnorm_qk=False,
        ring_degree=2, chunk_lens=_even(256, 2), q_start=0, q_len=256, seed=1001,
        note="Q=256 vs 2 KV chunks of 128, fp32 in, scale 1/sqrt(64)"),
    "flux": Workload(
        name="flux", B=1, H=24, S=4608, d=128, dtype="bf16", rmsnorm_qk=True,
        ring_degree=2, chunk_lens=_even(4608, 2), q_start=0, q_len=2304, seed=1002,
        note="FLUX.1-dev 1024x1024 joint attention, 512 text + 4096 image tokens, ring-2 rank-0 share"),
    "cogvideox": Workload(
        name="cogvideox", B=1, H=48, S=17776, d=64, dtype="bf16", rmsnorm_qk=False,
        ring_degree=1, chunk_lens=(17776,), q_start=0, q_len=17776, seed=1003,
        ulysses_degree=2, ulysses_group=0,
        note="CogVideoX-5b, 226 text + 13x30x45 video tokens, Ulysses-2 share: seq-shard -> 24-head permute"),
    "mochi": Workload(
        name="mochi", B=1, H=24, S=44776, d=128, dtype="bf16", rmsnorm_qk=True,
        ring_degree=4, chunk_lens=_even(44776, 4), q_start=0, q_len=11194, seed=1004,
        note="Mochi-1 256 text + 28x30x53 video tokens, ring-4 rank-0 share"),
    "ring_anything": Workload(
        name="ring_anything", B=2, H=24, S=4608, d=128, dtype="bf16", rmsnorm_qk=False,
        ring_degree=5, chunk_lens=(922, 922, 922, 921, 921), q_start=0, q_len=922, seed=1005,
        note="uneven 5-way Ring Anything split, CFG batch of 2, rank-0 share"),
}

ORDER = ("tiny", "flux", "cogvideox", "mochi", "ring_anything")


# ----------------------------------------------------------------------------
# bfloat16 helpers (bit-level, numpy only)
# ----------------------------------------------------------------------------

def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------

def _rmsnorm_rows(x: np.ndarray) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(RMS_EPS))).astype(np.float32)


@dataclass
class Inputs:
    """Token-major tensors [B, S, H, d].

    ``q``/``k``/``v`` are float32 arrays holding exactly the values handed to the
    library (already bf16-representable for bf16 workloads).  ``*_bits`` hold
    the bf16 bit patterns (None for fp32 workloads).
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None


def draw_bshd(rng: np.random.Generator, B: int, S: int, H: int, d: int) -> np.ndarray:
    return rng.standard_normal((B, S, H, d), dtype=np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    q = draw_bshd(rng, wl.B, wl.S, wl.H, wl.d)
    k = draw_bshd(rng, wl.B, wl.S, wl.H, wl.d)
    v = draw_bshd(rng, wl.B, wl.S, wl.H, wl.d)
    if wl.rmsnorm_qk:
        q = _rmsnorm_rows(q)
        k = _rmsnorm_rows(k)
    if wl.dtype == "fp32":
        return Inputs(wl, q, k, v)
    qb, kb, vb = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
    return Inputs(wl, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), qb, kb, vb)


def random_bhsd(seed: int, shape, dtype: str = "bf16", scale: float = 1.0):
    """Small helper for tests: N(0, scale^2) of ``shape``.

    Returns (values_f32, storage): storage is None for "fp32", the bf16 bit
    patterns (uint16, nearest-even) for "bf16", and the float16 array
    (numpy's nearest-even cast) for "fp16"; values_f32 holds the rounded values.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    if dtype == "fp32":
        return x, None
    if dtype == "fp16":
        h = x.astype(np.float16)
        return h.astype(np.float32), h
    b = bf16_round_bits(x)
    return bf16_bits_to_f32(b), b


def to_bhsd(x: np.ndarray) -> np.ndarray:
    """[B, S, H, d] -> contiguous [B, H, S, d] (layout only)."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)))


def chunk_offsets(chunk_lens) -> Tuple[int, ...]:
    offs, o = [], 0
    for n in chunk_lens:
        offs.append(o)
        o += n
    return tuple(offs)


def sample_rows(n_rows: int, seed: int, n_random: int = 256, tiles=(128, 256), upto: int = 1024):
    """Deterministic query-row sample for shares too big for the oracle in full.

    First and last 64 rows, both sides of every 128/256 tile boundary in the first
    ``upto`` rows, and ``n_random`` seeded random rows; sorted and unique.
    """
    rows = set(range(min(64, n_rows)))
    rows |= set(range(max(0, n_rows - 64), n_rows))
    for t in tiles:
        for b in range(t, min(upto, n_rows), t):
            rows |= {b - 1, b}
    rng = np.random.Generator(np.random.PCG64(seed))
    rows |= set(int(r) for r in rng.integers(0, n_rows, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < n_rows), dtype=np.int64)
