"""Helpers shared by the GPU tests: device transfer and the parity bars."""
from __future__ import annotations

import sys

import numpy as np
import torch

from context_attention_diffusion_non_amd import workloads as W

DEV = "cuda:0"

# GPU-vs-oracle bars for the attention output and LSE
MAX_ABS_OUT = 2e-2
MEAN_ABS_OUT = 2e-3
MAX_ABS_LSE = 1e-3
# extra guard: an all-zero output would pass the absolute bars at these tiny
# output magnitudes, so the relative Frobenius error is bounded as well
REL_FROB_OUT = 1e-2
# GPU chunked (ring) vs GPU unsplit, both fp32 out
CHUNKED_VS_UNSPLIT = 1e-3

BF16_BARS = dict(max_abs_out=MAX_ABS_OUT, mean_abs_out=MEAN_ABS_OUT, rel_frob=REL_FROB_OUT, max_abs_lse=MAX_ABS_LSE)
# fp16 inputs: P is rounded to fp16 (relative 2^-11, 8x finer than bf16) and an
# fp16 output of |o| < 8 rounds by at most 2^-9; the bars are those two
# contributions with margin.  The LSE keeps the bf16 path's bar (fp32 row sums).
FP16_BARS = dict(max_abs_out=4e-3, mean_abs_out=4e-4, rel_frob=2e-3, max_abs_lse=MAX_ABS_LSE)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def rand_bf16(seed: int, shape, scale: float = 1.0):
    """(float64 values, device bf16 tensor) of N(0, scale^2) rounded to bf16."""
    vals, bits = W.random_bhsd(seed, shape, "bf16", scale)
    return vals.astype(np.float64), bits_to_dev(bits)


def rand_f16(seed: int, shape, scale: float = 1.0):
    """(float64 values, device fp16 tensor) of N(0, scale^2) rounded to fp16."""
    vals, h = W.random_bhsd(seed, shape, "fp16", scale)
    return vals.astype(np.float64), torch.from_numpy(np.ascontiguousarray(h)).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity(out: torch.Tensor, lse: torch.Tensor, ref_out: np.ndarray, ref_lse: np.ndarray, what: str,
           bars: dict = BF16_BARS) -> dict:
    o = to_np(out)
    l = to_np(lse)
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    err = np.abs(o - ref_out)
    max_o, mean_o = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref_out))
    rel = float(np.linalg.norm(o - ref_out) / nrm) if nrm > 0 else float(np.linalg.norm(o))
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(l)), f"{what}: -inf pattern of lse differs"
    assert np.all(l[~fin] == ref_lse[~fin]), f"{what}: non-finite lse values differ"
    max_l = float(np.abs(l[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    log(f"[parity] {what}: max|dout|={max_o:.3e} mean|dout|={mean_o:.3e} rel_frob={rel:.3e} max|dlse|={max_l:.3e}")
    assert max_o <= bars["max_abs_out"], f"{what}: max abs out error {max_o}"
    assert mean_o <= bars["mean_abs_out"], f"{what}: mean abs out error {mean_o}"
    assert rel <= bars["rel_frob"], f"{what}: relative Frobenius error {rel}"
    assert max_l <= bars["max_abs_lse"], f"{what}: max abs lse error {max_l}"
    return dict(max_abs_out=max_o, mean_abs_out=mean_o, rel_frob=rel, max_abs_lse=max_l)
