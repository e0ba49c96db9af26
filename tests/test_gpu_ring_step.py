"""GPU parity of the one-launch ring step against the fp64 oracle.

cpattn_ring_fwd runs a whole ring step as one launch: the (query tile, key
tile) units of all chunks are split into equal contiguous ranges, one
workgroup each, chunk boundaries are closed in registers by the log-sum-exp
identity, and query tiles cut by a range boundary are written as pieces and
merged in key order by a second small launch.  The cases here are chosen (and
checked, with the plan written out below from the library's documented
rule) so that cuts fall inside a chunk and on a chunk boundary, pieces span
chunk boundaries and a query tile is cut into three or more pieces; empty chunks and chunk tails shorter than a key tile are among
them.  Every case is compared with oracle.ring_attention (the per-chunk
attention and the chunk-ordered LSE merge), with the GPU's unsplit attention
(chunked vs unsplit), and with itself on a second run (bitwise)."""
import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import CHUNKED_VS_UNSPLIT, log, parity, rand_bf16, to_np

pytestmark = pytest.mark.gpu

KEYS = 64       # keys per tile
MIN_TILES = 8   # fewest key tiles per workgroup


def pieces(B, H, Sq, d, lens):
    """(T, chunk tile starts, {query tile: [(g0, g1), ...]}) of the one-launch ring step as
    the library plans it.  A step whose 128-row query tiles fit one round of four-wave
    workgroups runs 256-row tiles whole; otherwise 256-row tiles run whole in rounds of S
    eight-wave workgroups and the L leftover tiles are cut at key tile a = round(L T / S) into a head
    (one workgroup each) and a tail, the tails laid end to end and split into S - L equal
    contiguous ranges."""
    starts, T = [], 0
    for n in lens:
        if n > 0:
            starts.append(T)
            T += -(-n // KEYS)
    slots4, slots8 = (512, 256) if d == 128 else (1024, 512)
    q4, q8 = B * H * -(-Sq // 128), B * H * -(-Sq // 256)
    if q4 <= slots4 and q8 <= slots8:
        return T, starts, {j: [(0, T)] for j in range(q8)}
    Q = q8                      # split steps run 256-row tiles too, on the eight-wave slots
    S = min(slots8, max(1, -(-(Q * T) // MIN_TILES)))
    R, L = divmod(Q, S)
    a = min(T, (2 * L * T + S) // (2 * S)) if L else 0
    out = {j: [(0, T)] for j in range(R * S)}
    for i in range(L):
        out[R * S + i] = [(0, a)] if a else []
    if L:
        per, rem = divmod(L * (T - a), S - L)
        begins = [t * per + min(t, rem) for t in range(S - L + 1)]
        for t in range(S - L):
            u = begins[t]
            while u < begins[t + 1]:
                i, g = divmod(u, T - a)
                g1 = min(T - a, g + begins[t + 1] - u)
                out[R * S + i].append((a + g, a + g1))
                u += g1 - g
    return T, starts, out


def coverage(B, H, Sq, d, lens):
    T, starts, ps = pieces(B, H, Sq, d, lens)
    cuts = [g1 for p in ps.values() if len(p) > 1 for (_, g1) in p[:-1]]
    crossing = any(any(g0 < s < g1 for s in starts) for p in ps.values() if len(p) > 1 for (g0, g1) in p)
    return dict(inside=any(c not in starts for c in cuts), on_boundary=any(c in starts for c in cuts),
                crossing=crossing, most_pieces=max(len(p) for p in ps.values()))


CASES = [  # B, H, Sq, d, chunk lengths
    # whole 256-row tiles in one round (chunk closes in registers, no pieces)
    (1, 1, 16, 128, (300, 500, 224)),
    (2, 3, 150, 128, (0, 129, 0, 127, 65)),
    (1, 2, 300, 64, (2000,)),
    # more 128-row tiles than one round: rounds, then heads and split tails
    (1, 600, 40, 128, (448, 3, 0, 512, 61)),
    (2, 300, 40, 128, (999, 777)),
    (1, 1100, 40, 64, (2000,)),
    (1, 700, 200, 128, (129, 127, 65)),
    (1, 513, 16, 128, (512, 512)),
]


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


def test_cases_cover_the_split_kinds():
    cov = [coverage(*c) for c in CASES]
    assert any(c["inside"] for c in cov)
    assert any(c["on_boundary"] for c in cov)
    assert any(c["crossing"] for c in cov)
    assert any(c["most_pieces"] >= 3 for c in cov)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}Sq{c[2]}d{c[3]}-{'-'.join(map(str, c[4]))}")
def test_ring_step_splits(case):
    B, H, Sq, d, lens = case
    cov = coverage(*case)
    log(f"[case] one-launch ring B={B} H={H} Sq={Sq} d={d} lens={lens} {cov}")
    skv = sum(lens)
    seed = 9000 + Sq + skv + d
    qv, q = rand_bf16(seed, (B, H, Sq, d))
    kv, k = rand_bf16(seed + 1, (B, H, skv, d))
    vv, v = rand_bf16(seed + 2, (B, H, skv, d))
    out, lse = ops.ring_fwd(q, k, v, len(lens), list(lens), out_dtype=torch.bfloat16)
    out2, lse2 = ops.ring_fwd(q, k, v, len(lens), list(lens), out_dtype=torch.bfloat16)
    r32, l32 = ops.ring_fwd(q, k, v, len(lens), list(lens), out_dtype=torch.float32)
    f32, fl32 = ops.block_fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)
    d_o = (r32 - f32).abs().max().item()
    d_l = (l32 - fl32).abs().max().item()
    log(f"[parity] chunked-vs-unsplit fp32: out={d_o:.3e} lse={d_l:.3e}")
    assert d_l <= CHUNKED_VS_UNSPLIT
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    e_ring = float(np.abs(to_np(r32) - ro).max())
    e_full = float(np.abs(to_np(f32) - ro).max())
    log(f"[parity] fp32 max|dout| vs oracle: chunked {e_ring:.3e}, unsplit {e_full:.3e}")
    # The bf16 rounding of P (relative 2^-8 per weight) differs between two correct
    # evaluations, so the difference of two outputs shrinks only as 1/sqrt(keys): near
    # 1e-3 at a thousand keys.  The 1e-3 bar holds from 2000 keys on; at every size the
    # chunked result's own error may not exceed the unsplit one's by more than that noise.
    if skv >= 2000:
        assert d_o <= CHUNKED_VS_UNSPLIT
    assert e_ring <= 1.5 * e_full + 5e-5
    parity(out, lse, ro, rl, f"one-launch ring {case} bf16")
    parity(r32, l32, ro, rl, f"one-launch ring {case} fp32")


def test_more_chunks_than_one_launch_takes():
    """130 chunks: past the one-launch chunk table, the step runs one launch per chunk with the
    fp32 accumulator in the workspace."""
    lens = [7, 0, 64, 1] * 32 + [100, 30]
    log(f"[case] ring with {len(lens)} chunks")
    skv = sum(lens)
    qv, q = rand_bf16(9501, (1, 2, 140, 128))
    kv, k = rand_bf16(9502, (1, 2, skv, 128))
    vv, v = rand_bf16(9503, (1, 2, skv, 128))
    out, lse = ops.ring_fwd(q, k, v, len(lens), lens, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    parity(out, lse, ro, rl, "130-chunk ring")


@pytest.mark.parametrize("B,H,Sq", [(1, 2, 300), (1, 300, 40)], ids=["whole-tiles", "rounds-and-cuts"])
def test_128_chunks_in_one_launch(B, H, Sq):
    """128 non-empty chunks of uneven length (1 to 65 keys, so most chunks are one partial key
    tile): the largest chunk table one launch takes, run whole and in rounds with cut tiles."""
    lens = [3, 64, 65, 1] * 32
    T, _, ps = pieces(B, H, Sq, 128, lens)
    cut = any(p != [(0, T)] for p in ps.values())
    assert cut == (H == 300)
    log(f"[case] ring with 128 chunks, B={B} H={H} Sq={Sq} ({'cut tiles' if cut else 'whole tiles'})")
    skv = sum(lens)
    qv, q = rand_bf16(9701 + H, (B, H, Sq, 128))
    kv, k = rand_bf16(9702 + H, (B, H, skv, 128))
    vv, v = rand_bf16(9703 + H, (B, H, skv, 128))
    out, lse = ops.ring_fwd(q, k, v, len(lens), lens, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    parity(out, lse, ro, rl, f"128-chunk ring H={H}")


def test_no_split_needs_no_workspace():
    """A step that runs every query tile whole writes no pieces: no workspace is needed."""
    B, H, Sq, d, lens = 1, 2, 256, 128, (256, 256)
    T, _, ps = pieces(B, H, Sq, d, lens)
    assert all(p == [(0, T)] for p in ps.values())
    log("[case] ring without split tiles, no workspace")
    qv, q = rand_bf16(9601, (B, H, Sq, d))
    kv, k = rand_bf16(9602, (B, H, sum(lens), d))
    vv, v = rand_bf16(9603, (B, H, sum(lens), d))
    out = torch.empty(B, H, Sq, d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(B, H, Sq, device=q.device)
    st = _lib.lib().cpattn_ring_fwd(ops._ptr(q), ops._ptr(k), ops._ptr(v), ops._ptr(out), ops._ptr(lse), B, H, Sq,
                                    sum(lens), d, 0.0, len(lens), (ops.ctypes.c_int64 * 2)(*lens), None, 0,
                                    _lib.BF16, _lib.BF16, ops._stream(q))
    _lib.check(st)
    torch.cuda.synchronize()
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    parity(out, lse, ro, rl, "ring without split tiles")
