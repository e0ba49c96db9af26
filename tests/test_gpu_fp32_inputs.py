"""GPU parity for fp32 inputs (CPATTN_FP32), the element type of the tiny ring
share.  The MFMA path rounds fp32 q/k/v to bf16 (RNE) as it stages them, so the
graded oracle sees the bf16-rounded values.  The raw-fp32 oracle is asserted
too: the output at the same bars, the LSE within the bound that the bf16
staging of q and k implies.  Shapes put the query and key tails off the 64-key tile and
the 32-row wave block, at d = 64 and 128, with fp32 and bf16 outputs, ragged
ring chunks (empty and 3-key chunks among them) and a K/V window addressed in
place inside a larger buffer (kv_ld > Skv)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from context_attention_diffusion_non_amd import workloads as W
from tests.gpu_util import DEV, f32_to_dev, log, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


def _f32(seed, shape):
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32)
    return x, f32_to_dev(x)


def _r(x):
    """The bf16-rounded values the kernel consumes, in fp64."""
    return W.bf16_round(x).astype(np.float64)


SHAPES = [(2, 3, 129, 63, 128), (1, 2, 300, 200, 128), (1, 2, 127, 65, 64), (3, 1, 257, 129, 64),
          (1, 1, 33, 777, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_block_fwd_fp32_inputs_ragged(shape, out_dtype):
    B, H, Sq, Skv, d = shape
    log(f"[case] fp32-in block_fwd B={B} H={H} Sq={Sq} Skv={Skv} d={d} out={out_dtype}")
    seed = 7000 + Sq + Skv + d
    q, qd = _f32(seed, (B, H, Sq, d))
    k, kd = _f32(seed + 1, (B, H, Skv, d))
    v, vd = _f32(seed + 2, (B, H, Skv, d))
    out, lse = ops.block_fwd(qd, kd, vd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(_r(q), _r(k), _r(v))
    parity(out, lse, ro, rl, f"fp32-in block_fwd {shape} {out_dtype}")


@pytest.mark.parametrize("lens", [(129, 127, 65, 3), (0, 64, 0, 100), (200, 1)], ids=str)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32out", "bf16out"])
def test_ring_fp32_inputs_uneven_chunks(lens, d, out_dtype):
    log(f"[case] fp32-in ring lens={lens} d={d} out={out_dtype}")
    skv = sum(lens)
    q, qd = _f32(7100 + d, (2, 2, 150, d))
    k, kd = _f32(7101 + d, (2, 2, skv, d))
    v, vd = _f32(7102 + d, (2, 2, skv, d))
    out, lse = ops.ring_fwd(qd, kd, vd, len(lens), list(lens), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.ring_attention(_r(q), _r(k), _r(v), lens)
    parity(out, lse, ro, rl, f"fp32-in ring {lens} d={d} {out_dtype}")


@pytest.mark.parametrize("d", [64, 128])
def test_block_fwd_fp32_kv_window_in_place(d):
    """An fp32 chunk addressed inside its parent K/V buffer: kv_ld = 300 rows, keys 50 .. 172."""
    B, H, Sq, ld, off, n = 2, 3, 70, 300, 50, 123
    log(f"[case] fp32-in kv_ld window d={d}")
    q, qd = _f32(7200 + d, (B, H, Sq, d))
    k, kd = _f32(7201 + d, (B, H, ld, d))
    v, vd = _f32(7202 + d, (B, H, ld, d))
    out = torch.empty(B, H, Sq, d, device=DEV)
    lse = torch.empty(B, H, Sq, device=DEV)
    st = _lib.lib().cpattn_block_fwd(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr() + off * d * 4),
                                     ctypes.c_void_p(vd.data_ptr() + off * d * 4), ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(lse.data_ptr()), B, H, Sq, n, ld, d, 0.0, _lib.FP32, _lib.FP32,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(_r(q), _r(k[:, :, off:off + n]), _r(v[:, :, off:off + n]))
    parity(out, lse, ro, rl, f"fp32-in kv_ld window d={d}")


def test_tiny_share_against_raw_fp32_oracle():
    """The tiny ring share (fp32 in and out) against the oracle on the seeded fp32 inputs as
    they are, not rounded.  The output meets the bf16 bars as they stand.  The LSE moves with
    the bf16 staging of q and k: log-sum-exp is 1-Lipschitz in the max norm of the scores, so
    |LSE(rounded) - LSE(raw)| <= max_j |s_j(rounded) - s_j(raw)| per row, which the test computes
    exactly in fp64 from the two input sets and allows on top of 2e-5 of kernel rounding."""
    wl = W.WORKLOADS["tiny"]
    log("[case] tiny ring-2 vs the raw-fp32 oracle")
    x = W.make_inputs(wl)
    q, k, v = (f32_to_dev(W.to_bhsd(t)) for t in (x.q, x.k, x.v))
    out, lse = ops.ring_fwd(q, k, v, wl.ring_degree, list(wl.chunk_lens))
    torch.cuda.synchronize()
    raw = [W.to_bhsd(t).astype(np.float64) for t in (x.q, x.k, x.v)]
    rnd = [_r(W.to_bhsd(t)) for t in (x.q, x.k, x.v)]
    ro, rl = oracle.ring_attention(*raw, wl.chunk_lens)
    o = out.cpu().numpy().astype(np.float64)
    err = np.abs(o - ro)
    scale = 1.0 / np.sqrt(wl.d)
    ds = np.abs(rnd[0] @ rnd[1].transpose(0, 1, 3, 2) - raw[0] @ raw[1].transpose(0, 1, 3, 2)) * scale
    bound = ds.max(axis=-1) + 2e-5
    dl = np.abs(lse.cpu().numpy().astype(np.float64) - rl)
    log(f"[parity] tiny vs raw fp32: max|dout|={err.max():.3e} mean={err.mean():.3e} "
        f"max|dlse|={dl.max():.3e} (largest fraction of its per-row bound {(dl / bound).max():.3f})")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.all(dl <= bound)
