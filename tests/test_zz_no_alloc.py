"""cpattn_ring_fwd_noalloc, the allocation-free ring step, against cpattn_ring_fwd.

Both run the same kernels and the same launch plan, so the outputs must agree
bit for bit; here on shapes whose steps cut query tiles (so the library's own
scratch carries the pieces) and on one that runs whole tiles, two calls in a
row with the second smaller than the first (the scratch keeps the first call's
contents, which the second must never read), under HIP graph capture, and on
the refusal past 128 chunks."""
import ctypes

import pytest
import torch

from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import log, rand_bf16

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, Sq, skv, d):
    _, q = rand_bf16(seed, (B, H, Sq, d))
    _, k = rand_bf16(seed + 1, (B, H, skv, d))
    _, v = rand_bf16(seed + 2, (B, H, skv, d))
    return q, k, v


def _both(q, k, v, lens, out_dtype):
    B, H, Sq, d = q.shape
    ref_o, ref_l = ops.ring_fwd(q, k, v, len(lens), list(lens), out_dtype=out_dtype)
    out = torch.full((B, H, Sq, d), float("nan"), dtype=out_dtype, device=q.device)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=q.device)
    ops.ring_fwd_noalloc(q, k, v, len(lens), list(lens), out=out, lse=lse)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                       b.view(torch.int16) if b.dtype != torch.float32 else b)


def test_scratch_size_is_stated(lib_path):
    assert _lib.lib().cpattn_ring_fwd_noalloc_scratch_bytes() == 68157440


@pytest.mark.parametrize("d", [128, 64])
def test_noalloc_matches_ring_fwd_twice_second_smaller(lib_path, d):
    # 600 (d = 128) / 1100 (d = 64) planes: more 128-row tiles than a round of workgroups,
    # so the step cuts the leftover tiles and writes pieces to the scratch; the second call
    # has fewer planes, fewer rows and other chunk lengths
    H1, H2 = (600, 530) if d == 128 else (1100, 1040)
    for n, (H, Sq, lens, od) in enumerate([(H1, 40, (448, 3, 0, 512, 61), torch.bfloat16),
                                          (H2, 30, (300, 200), torch.float32)]):
        log(f"[case] noalloc call {n + 1}: H={H} Sq={Sq} d={d} lens={lens}")
        q, k, v = _inputs(7700 + 10 * n + d, 1, H, Sq, sum(lens), d)
        ref_o, ref_l, out, lse = _both(q, k, v, lens, od)
        assert _same(ref_o, out) and torch.equal(ref_l, lse), f"call {n + 1} differs from cpattn_ring_fwd"


def test_noalloc_whole_tiles(lib_path):
    log("[case] noalloc, whole tiles")
    q, k, v = _inputs(7800, 2, 3, 300, 700, 128)
    ref_o, ref_l, out, lse = _both(q, k, v, (350, 350), torch.bfloat16)
    assert _same(ref_o, out) and torch.equal(ref_l, lse)


def test_noalloc_under_graph_capture(lib_path):
    """The caller it is for: a captured step (pieces of cut tiles in the library's scratch, then
    the fixup launch) replayed after eager work, bit for bit the eager call each time, also on
    inputs rewritten in place."""
    H, Sq, lens, d = 600, 40, (448, 3, 0, 512, 61), 128
    log(f"[case] noalloc under graph capture: H={H} Sq={Sq} d={d} lens={lens}")
    q, k, v = _inputs(8100, 1, H, Sq, sum(lens), d)
    out = torch.empty(1, H, Sq, d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(1, H, Sq, dtype=torch.float32, device=q.device)

    def call():
        ops.ring_fwd_noalloc(q, k, v, len(lens), list(lens), out=out, lse=lse)

    call()  # the first call on the device looks the scratch up, outside the capture
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(5.0)
        lse.fill_(-1.0)
        ops.ring_fwd(q[:, :7], k[:, :7], v[:, :7], len(lens), list(lens))  # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, ref_o) and torch.equal(lse, ref_l), f"replay {i} differs from the eager call"
    q2, k2, v2 = _inputs(8200, 1, H, Sq, sum(lens), d)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    call()
    torch.cuda.synchronize()
    ref2_o, ref2_l = out.clone(), lse.clone()
    out.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert _same(out, ref2_o) and torch.equal(lse, ref2_l), "replay on new inputs differs"


def test_noalloc_refuses_more_than_128_chunks(lib_path):
    q, k, v = _inputs(7900, 1, 1, 16, 130, 128)
    out = torch.empty(1, 1, 16, 128, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(1, 1, 16, device=q.device)
    with pytest.raises(_lib.CpattnError) as e:
        ops.ring_fwd_noalloc(q, k, v, 130, [1] * 130, out=out, lse=lse)
    assert e.value.name == "CPATTN_ERR_DEGREE" and "at most 128" in str(e.value)
