"""Unified attention (Ulysses regroup + ring over the regrouped segments) through
the C ABI: every rank's share against the fp64 oracle's share, and the pages'
own correctness example on 2 x 2 and 2 x 4 grids, each rank's output regrouped
back by token and compared with unsplit attention at the pages' tolerance."""
import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import BF16_BARS, DEV, FP16_BARS, log, parity, rand_bf16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


def _shards(full_vals, full_dev, W):
    """[B, S, H, d] full sequence -> [W, B, S/W, H, d] sequence shards (values, device tensor)."""
    B, S, H, d = full_vals.shape
    vals = np.ascontiguousarray(full_vals.reshape(B, W, S // W, H, d).transpose(1, 0, 2, 3, 4))
    dev = full_dev.reshape(B, W, S // W, H, d).permute(1, 0, 2, 3, 4).contiguous()
    return vals, dev


MESHES = [(2, 2, 37, 64, torch.bfloat16), (1, 2, 64, 128, torch.float32), (2, 1, 50, 64, torch.bfloat16),
          (3, 2, 29, 128, torch.bfloat16), (2, 3, 16, 64, torch.float32)]


@pytest.mark.parametrize("R,U,S_loc,d,out_dtype", MESHES, ids=lambda x: str(x))
def test_unified_every_rank_vs_oracle(R, U, S_loc, d, out_dtype):
    B, H = 2, 2 * U
    W = R * U
    log(f"[case] unified R={R} U={U} S_loc={S_loc} d={d} out={out_dtype}")
    shards = []
    for i in range(3):
        vals, dev = rand_bf16(300 + 10 * R + U + i, (B, W * S_loc, H, d))
        shards.append(_shards(vals, dev, W))
    (qv, q), (kv, k), (vv, v) = shards
    for rr in range(R):
        for ur in range(U):
            out, lse = ops.unified_fwd(q, k, v, R, U, rr, ur, out_dtype=out_dtype)
            torch.cuda.synchronize()
            ro, rl = oracle.unified_rank_share(qv, kv, vv, R, U, rr, ur)
            parity(out, lse, ro, rl, f"unified {R}x{U} rank ({rr},{ur}) {out_dtype}", BF16_BARS)


@pytest.mark.parametrize("R,U", [(2, 2), (2, 4)])
def test_pages_example_unified(pages_example, R, U):
    """The pages' check: each rank's output rows (its own tokens, every head)
    after the reverse regroup equal unsplit attention sliced to those rows,
    within rtol 1e-5 and atol 1e-3 * world_size."""
    ex = pages_example
    W = R * U
    S = ex["S"]
    S_loc = S // W
    atol, rtol = 1e-3 * W, 1e-5
    to_shards = lambda t: t.permute(0, 2, 1, 3).reshape(2, W, S_loc, 24, 64).permute(1, 0, 2, 3, 4).contiguous()
    q, k, v = (to_shards(ex[n]) for n in ("q", "k", "v"))
    ref = np.transpose(ex["ref_out"], (0, 2, 1, 3)).reshape(2, W, S_loc, 24, 64).transpose(1, 0, 2, 3, 4)
    ref_lse = np.transpose(ex["ref_lse"], (0, 2, 1)).reshape(2, W, S_loc, 24).transpose(1, 0, 2, 3)
    worst = 0.0
    for rr in range(R):
        log(f"[case] pages example unified {R}x{U} ulysses group {rr}")
        outs, lses = [], []
        for ur in range(U):
            o, l = ops.unified_fwd(q, k, v, R, U, rr, ur)
            outs.append(o)
            lses.append(l)
        # reverse regroup inside the Ulysses group: [U, B, H/U, S/R, d] -> [U, B, S_loc, H, d]
        back = ops.ulysses_permute(torch.stack(outs), U, -1, 1)
        back_lse = ops.ulysses_permute(torch.stack(lses).unsqueeze(-1), U, -1, 1)[..., 0]
        torch.cuda.synchronize()
        assert back.dtype == torch.float16
        for ur in range(U):
            w = rr * U + ur
            o = to_np(back[ur])
            err = np.abs(o - ref[w])
            worst = max(worst, float(err.max()))
            assert (err - (atol + rtol * np.abs(ref[w]))).max() <= 0, f"rank {w}: max|dout| {err.max()}"
            assert np.abs(to_np(back_lse[ur]) - ref_lse[w]).max() <= 1e-3, f"rank {w}: lse"
            assert np.abs(o - ref[w]).mean() <= FP16_BARS["mean_abs_out"]
    log(f"[parity] pages example unified {R}x{U}: max|dout|={worst:.3e} (atol {atol:.0e})")
