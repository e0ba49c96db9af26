"""Ulysses Anything regroup through the C ABI: bit-exact against the oracle for
uneven sequence shards and head groups (the FLUX 1008x1008 sequence of 4481
tokens that no even split admits, a 5-way split of 24 heads, odd row sizes,
empty shards), both directions, and the regroup -> attention -> reverse
regroup composition against unsplit attention."""
import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import BF16_BARS, DEV, log, parity, rand_bf16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


_NP = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}
_TORCH = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
_VIEW = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}


CASES = [  # B, H, d, elem_bytes, seq_lens, head_lens
    (1, 24, 128, 2, oracle.even_split(4481, 2), [12, 12]),
    (2, 24, 64, 2, oracle.even_split(4481, 5), oracle.even_split(24, 5)),
    (1, 25, 64, 2, [34, 33, 33], [9, 8, 8]),
    (2, 7, 7, 2, [5, 0, 6, 4], [2, 2, 0, 3]),
    (1, 6, 3, 4, [9, 10], [4, 2]),
    (3, 5, 16, 1, [1, 2, 3], [1, 3, 1]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}d{c[2]}eb{c[3]}P{len(c[4])}")
def test_anything_permute_bit_exact(case):
    B, H, d, eb, seq_lens, head_lens = case
    P, S = len(seq_lens), sum(seq_lens)
    log(f"[case] anything permute B={B} H={H} d={d} eb={eb} seq={seq_lens} heads={head_lens}")
    r = np.random.Generator(np.random.PCG64(S * 31 + H))
    shards = [r.integers(0, np.iinfo(_NP[eb]).max, size=(B, n, H, d), dtype=_NP[eb]) for n in seq_lens]
    packed = np.concatenate([s.reshape(-1) for s in shards])
    x = torch.from_numpy(packed.view(_VIEW[eb])).to(DEV)
    groups = []
    for g in range(P):
        out = ops.ulysses_anything_permute(x, B, H, d, seq_lens, head_lens, g, 0)
        ref = oracle.anything_seq_to_head(shards, head_lens, g)
        assert np.array_equal(out.cpu().numpy().view(_NP[eb]).reshape(ref.shape), ref), f"group {g}"
        groups.append(ref)
    allg = ops.ulysses_anything_permute(x, B, H, d, seq_lens, head_lens, -1, 0)
    ref_all = np.concatenate([g_.reshape(-1) for g_ in groups])
    assert np.array_equal(allg.cpu().numpy().view(_NP[eb]), ref_all), "all groups"
    # reverse: every group at once, and one group into a buffer whose other heads must stay
    back = ops.ulysses_anything_permute(allg, B, H, d, seq_lens, head_lens, -1, 1)
    assert np.array_equal(back.cpu().numpy().view(_NP[eb]), packed), "round trip"
    g1 = max(range(P), key=lambda i: head_lens[i])
    y = torch.from_numpy(groups[g1].reshape(-1).view(_VIEW[eb])).to(DEV)
    base = torch.full((packed.size,), 7, dtype=_TORCH[eb], device=DEV)
    one = ops.ulysses_anything_permute(y, B, H, d, seq_lens, head_lens, g1, 1, out=base)
    torch.cuda.synchronize()
    got = one.cpu().numpy().view(_NP[eb])
    off = 0
    h0 = sum(head_lens[:g1])
    for n in seq_lens:
        blk = got[off:off + B * n * H * d].reshape(B, n, H, d)
        src = packed[off:off + B * n * H * d].reshape(B, n, H, d)
        assert np.array_equal(blk[:, :, h0:h0 + head_lens[g1]], src[:, :, h0:h0 + head_lens[g1]])
        mask = np.ones(H, bool)
        mask[h0:h0 + head_lens[g1]] = False
        assert np.all(blk[:, :, mask] == 7)
        off += B * n * H * d


def test_anything_attention_composition():
    """Regroup q, k, v into uneven head groups, attend every group over the whole
    sequence, regroup back: each rank's tokens match unsplit attention."""
    B, H, d = 1, 10, 64
    seq_lens, head_lens = oracle.even_split(1001, 3), oracle.even_split(H, 3)
    S = sum(seq_lens)
    log(f"[case] anything composition seq={seq_lens} heads={head_lens}")
    full = [rand_bf16(400 + i, (B, S, H, d)) for i in range(3)]
    off = np.concatenate([[0], np.cumsum(seq_lens)]).astype(int)
    packed = []
    for vals, dev in full:
        packed.append(torch.cat([dev[:, off[r]:off[r + 1]].reshape(-1) for r in range(3)]))
    outs = []
    for g in range(3):
        qg, kg, vg = (ops.ulysses_anything_permute(p, B, H, d, seq_lens, head_lens, g, 0) for p in packed)
        o, _ = ops.block_fwd(qg, kg, vg)
        outs.append(o.reshape(-1))
    back = ops.ulysses_anything_permute(torch.cat(outs), B, H, d, seq_lens, head_lens, -1, 1)
    torch.cuda.synchronize()
    qv, kv, vv = (np.transpose(f[0], (0, 2, 1, 3)) for f in full)
    ro, rl = oracle.attention(qv, kv, vv)                      # [B, H, S, d]
    ref = np.transpose(ro, (0, 2, 1, 3))                       # [B, S, H, d]
    got = to_np(back)
    o0 = 0
    for r in range(3):
        n = seq_lens[r]
        blk = got[o0:o0 + B * n * H * d].reshape(B, n, H, d)
        err = np.abs(blk - ref[:, off[r]:off[r + 1]])
        log(f"[parity] anything rank {r}: max|dout|={err.max():.3e} mean={err.mean():.3e}")
        assert err.max() <= BF16_BARS["max_abs_out"] and err.mean() <= BF16_BARS["mean_abs_out"]
        o0 += B * n * H * d
