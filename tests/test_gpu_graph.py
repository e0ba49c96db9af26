"""The library's calls under HIP graph capture.

A rank's ring step is a fixed sequence of launches on one stream with caller-owned
buffers, no allocation, no memset and no host synchronisation inside, so a caller
can capture it once and replay it. Each replay here runs after eager work and a
synchronisation, and must reproduce the eager result bit for bit, also after the
inputs are overwritten in place between replays."""
import pytest
import torch

from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import DEV, log, rand_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


def _inputs(seed, B, H, Sq, Skv, d):
    _, q = rand_bf16(seed, (B, H, Sq, d))
    _, k = rand_bf16(seed + 1, (B, H, Skv, d))
    _, v = rand_bf16(seed + 2, (B, H, Skv, d))
    return q, k, v


@pytest.mark.parametrize("convert_to_fp32", [True, False], ids=["fp32_partials", "bf16_partials"])
def test_ring_fwd_graph_replays_match_eager(convert_to_fp32):
    B, H, Sq, d = 2, 4, 300, 128
    lens = [129, 127, 65, 3]
    Skv = sum(lens)
    log(f"[case] ring_fwd graph replay B{B} H{H} Sq{Sq} chunks {lens} convert_to_fp32={convert_to_fp32}")
    q, k, v = _inputs(70, B, H, Sq, Skv, d)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    need = ops.ring_fwd_workspace_bytes(B, H, Sq, d, len(lens), torch.bfloat16) if convert_to_fp32 else 0
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)

    def call():
        ops.ring_fwd(q, k, v, len(lens), lens, out=out, lse=lse, workspace=ws, convert_to_fp32=convert_to_fp32)

    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(-3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: out differs from the eager call"
        assert torch.equal(lse, ref_lse), f"replay {i}: lse differs from the eager call"

    # new inputs written in place: the graph reads the live buffers
    q2, k2, v2 = _inputs(80, B, H, Sq, Skv, d)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    call()
    torch.cuda.synchronize()
    ref2_out, ref2_lse = out.clone(), lse.clone()
    assert not torch.equal(ref2_out, ref_out)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2_out), f"replay {i} on new inputs: out differs"
        assert torch.equal(lse, ref2_lse), f"replay {i} on new inputs: lse differs"


def test_permute_then_ring_graph_replays_match_eager():
    """A Ulysses share as one graph: regroup q, k and v (seq -> head), then the ring step."""
    P, S_loc, H, d = 2, 192, 8, 64
    log(f"[case] permute + ring_fwd graph replay P{P} S_loc{S_loc} H{H} d{d}")
    g_in = [rand_bf16(90 + i, (P, 1, S_loc, H, d))[1] for i in range(3)]
    heads = [torch.empty((1, H // P, P * S_loc, d), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    out = torch.empty((1, H // P, P * S_loc, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, H // P, P * S_loc), dtype=torch.float32, device=DEV)

    def call():
        for x, y in zip(g_in, heads):
            ops.ulysses_permute(x, P, group=0, direction=0, out=y)
        ops.ring_fwd(heads[0], heads[1], heads[2], 1, out=out, lse=lse)

    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(4):
        for y in heads:
            y.zero_()
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {i}: out differs from the eager call"
        assert torch.equal(lse, ref_lse), f"replay {i}: lse differs from the eager call"
