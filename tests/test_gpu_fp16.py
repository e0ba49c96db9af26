"""fp16 inputs through the C ABI against the fp64 oracle.

fp16 is the dtype of the pages' own correctness check (ParaAttention README,
unified attention example: fp16, B=2, H=24, S=4096, D=64) and of the Mochi
runs in the diffusers context-parallel page.  The kernel runs fp16 inputs on
the f16 MFMA with P rounded to fp16; partials and the merge stay fp32."""
import math

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import DEV, FP16_BARS, f32_to_dev, log, parity, rand_f16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


SHAPES = [  # B, H, Sq, Skv, d
    (1, 1, 1, 1, 64), (1, 2, 127, 65, 64), (2, 3, 129, 63, 128), (1, 2, 300, 200, 128),
    (1, 1, 256, 1000, 128), (1, 1, 33, 777, 64), (3, 1, 257, 129, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32out", "f16out", "bf16out"])
def test_block_fwd_fp16_ragged(shape, out_dtype):
    B, H, Sq, Skv, d = shape
    log(f"[case] fp16 block_fwd B={B} H={H} Sq={Sq} Skv={Skv} d={d} out={out_dtype}")
    seed = (hash(shape) & 0xFFFF) + 7
    qv, q = rand_f16(seed, (B, H, Sq, d))
    kv, k = rand_f16(seed + 1, (B, H, Skv, d))
    vv, v = rand_f16(seed + 2, (B, H, Skv, d))
    out, lse = ops.block_fwd(q, k, v, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(qv, kv, vv)
    # a bf16 destination adds its own rounding (2^-9 relative) on top of the fp16 path
    bars = dict(FP16_BARS, max_abs_out=2e-2, mean_abs_out=2e-3, rel_frob=1e-2) if out_dtype == torch.bfloat16 \
        else FP16_BARS
    parity(out, lse, ro, rl, f"fp16 block_fwd {shape} {out_dtype}", bars)


@pytest.mark.parametrize("lens", [(0, 64, 0, 100), (129, 127, 65, 3), (300, 301)], ids=str)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16], ids=["f32out", "f16out"])
def test_ring_fp16_uneven_chunks(lens, out_dtype):
    log(f"[case] fp16 ring lens={lens} out={out_dtype}")
    skv = sum(lens)
    qv, q = rand_f16(81, (2, 2, 150, 64))
    kv, k = rand_f16(82, (2, 2, skv, 64))
    vv, v = rand_f16(83, (2, 2, skv, 64))
    out, lse = ops.ring_fwd(q, k, v, len(lens), list(lens), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    parity(out, lse, ro, rl, f"fp16 ring {lens} {out_dtype}", FP16_BARS)


def test_fp16_scores_large_values():
    """fp16 inputs near the top of their range: scores of a few hundred after
    scaling must neither overflow nor lose the softmax (products accumulate in
    fp32; only P is stored in fp16, at most 2^8 by the exponent-base rule)."""
    log("[case] fp16 large values")
    qv, q = rand_f16(91, (1, 2, 130, 128), scale=30.0)
    kv, k = rand_f16(92, (1, 2, 300, 128), scale=30.0)
    vv, v = rand_f16(93, (1, 2, 300, 128), scale=100.0)
    out, lse = ops.block_fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(qv, kv, vv)
    o = to_np(out)
    assert np.all(np.isfinite(o))
    # values scale by 100: compare relative to that scale
    err = np.abs(o - ro).max() / 100.0
    lerr = np.abs(to_np(lse) - rl).max() / max(1.0, np.abs(rl).max())
    log(f"[parity] fp16 large: max|dout|/100={err:.3e} rel max|dlse|={lerr:.3e}")
    assert err <= FP16_BARS["max_abs_out"] and lerr <= 1e-5


def test_lse_merge_fp16_partials():
    log("[case] lse_merge fp16 partials")
    rows, d = 2049, 64
    r = np.random.Generator(np.random.PCG64(5))
    ao = r.standard_normal((rows, d)).astype(np.float32)
    bo = r.standard_normal((rows, d)).astype(np.float16)
    al = (r.standard_normal(rows) * 4).astype(np.float32)
    bl = (r.standard_normal(rows) * 4).astype(np.float32)
    bl[::5] = -np.inf
    acc_o, acc_l = f32_to_dev(ao), f32_to_dev(al)
    blk_o = torch.from_numpy(bo).to(DEV)
    blk_l = f32_to_dev(bl)
    ops.lse_merge(acc_o, acc_l, blk_o, blk_l)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(ao.astype(np.float64), al.astype(np.float64), bo.astype(np.float64),
                              bl.astype(np.float64))
    assert np.abs(to_np(acc_o) - ro).max() < 1e-5
    assert np.abs(to_np(acc_l) - rl).max() < 2e-6 * max(1.0, np.abs(rl).max())


@pytest.mark.parametrize("world_size", [2, 4])
def test_pages_example_ring_shares(pages_example, world_size):
    """Every rank's share of a ring of `world_size`: its query rows against the
    K/V chunks in the order the ring delivers them (own chunk first), output
    fp16; compared with the unsplit result sliced to the rank's rows with the
    pages' tolerance (rtol 1e-5, atol 1e-3 * world_size)."""
    ex = pages_example
    S, q, k, v = ex["S"], ex["q"], ex["k"], ex["v"]
    n = S // world_size
    atol, rtol = 1e-3 * world_size, 1e-5
    worst = 0.0
    for rank in range(world_size):
        log(f"[case] pages example ring ws={world_size} rank={rank}")
        order = [(rank + j) % world_size for j in range(world_size)]
        k_rot = torch.cat([k[:, :, c * n:(c + 1) * n] for c in order], dim=2).contiguous()
        v_rot = torch.cat([v[:, :, c * n:(c + 1) * n] for c in order], dim=2).contiguous()
        q_loc = q[:, :, rank * n:(rank + 1) * n].contiguous()
        out, lse = ops.ring_fwd(q_loc, k_rot, v_rot, world_size)
        torch.cuda.synchronize()
        ref = ex["ref_out"][:, :, rank * n:(rank + 1) * n]
        o = to_np(out)
        excess = np.abs(o - ref) - (atol + rtol * np.abs(ref))
        worst = max(worst, float(np.abs(o - ref).max()))
        assert excess.max() <= 0, f"rank {rank}: max|dout| {np.abs(o - ref).max()} over atol {atol}"
        lerr = np.abs(to_np(lse) - ex["ref_lse"][:, :, rank * n:(rank + 1) * n]).max()
        assert lerr <= 1e-3, f"rank {rank}: lse error {lerr}"
    log(f"[parity] pages example ring ws={world_size}: max|dout|={worst:.3e} (atol {atol:.0e})")


def test_pages_example_unsplit_fp16(pages_example):
    """The single-device baseline of the same check: one block, fp16 out."""
    ex = pages_example
    log("[case] pages example unsplit")
    out, lse = ops.block_fwd(ex["q"], ex["k"], ex["v"])
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    parity(out, lse, ex["ref_out"], ex["ref_lse"], "pages example unsplit fp16", FP16_BARS)
    err = np.abs(to_np(out) - ex["ref_out"])
    assert (err - (1e-3 + 1e-5 * np.abs(ex["ref_out"]))).max() <= 0
    assert math.isfinite(float(err.max()))
