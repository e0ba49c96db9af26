"""convert_to_fp32 ("Parallelism" API page, ContextParallelConfig): the default
keeps ring partials and their merges in fp32; False keeps the running output in
the output dtype between chunk steps.  Error study of both against the fp64
oracle over ring degrees 2, 4 and 8, plus edge cases of the 16-bit accumulator."""
import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import BF16_BARS, CHUNKED_VS_UNSPLIT, FP16_BARS, log, parity, rand_bf16, rand_f16, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded(lib_path):
    _lib.lib()


@pytest.fixture(scope="module")
def study_inputs():
    B, H, Sq, Skv, d = 1, 4, 512, 4096, 128
    qv, q = rand_bf16(500, (B, H, Sq, d))
    kv, k = rand_bf16(501, (B, H, Skv, d))
    vv, v = rand_bf16(502, (B, H, Skv, d))
    ro, rl = oracle.attention(qv, kv, vv)
    return dict(q=q, k=k, v=v, ro=ro, rl=rl, qv=qv, kv=kv, vv=vv)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_convert_to_fp32_error_study(study_inputs, n):
    x = study_inputs
    res = {}
    for c32 in (True, False):
        out, lse = ops.ring_fwd(x["q"], x["k"], x["v"], n, out_dtype=torch.bfloat16, convert_to_fp32=c32)
        torch.cuda.synchronize()
        res[c32] = parity(out, lse, x["ro"], x["rl"], f"ring N={n} bf16 out convert_to_fp32={c32}", BF16_BARS)
    log(f"[study] N={n}: mean|dout| fp32 partials {res[True]['mean_abs_out']:.3e}  "
        f"bf16 partials {res[False]['mean_abs_out']:.3e}  "
        f"(ratio {res[False]['mean_abs_out'] / res[True]['mean_abs_out']:.2f})")
    # rounding the running output at every step can only add error on average
    assert res[False]["mean_abs_out"] >= res[True]["mean_abs_out"]
    # the LSE never leaves fp32
    assert res[False]["max_abs_lse"] <= 1e-3


def test_convert_to_fp32_fp32_out_agrees(study_inputs):
    """With an fp32 output both settings keep the running output in fp32.  The default runs
    the step in one launch (each chunk's softmax based on the accumulator's LSE), False one
    launch per chunk (each chunk based on its own maximum), so P is rounded to bf16 against
    different bases: the two agree to the chunked-vs-unsplit bar, the LSE to fp32 rounding."""
    x = study_inputs
    a = ops.ring_fwd(x["q"], x["k"], x["v"], 4, out_dtype=torch.float32)
    b = ops.ring_fwd(x["q"], x["k"], x["v"], 4, out_dtype=torch.float32, convert_to_fp32=False)
    torch.cuda.synchronize()
    d_o = (a[0] - b[0]).abs().max().item()
    d_l = (a[1] - b[1]).abs().max().item()
    log(f"[parity] fp32 out, convert_to_fp32 True vs False: out={d_o:.3e} lse={d_l:.3e}")
    assert d_o <= CHUNKED_VS_UNSPLIT and d_l <= 1e-5
    parity(b[0], b[1], x["ro"], x["rl"], "ring N=4 fp32 out convert_to_fp32=False")


@pytest.mark.parametrize("lens", [(0, 64, 0, 100), (129, 127, 65, 3), (1, 1, 1, 1, 60)], ids=str)
def test_convert_to_fp32_false_uneven_and_empty(lens):
    skv = sum(lens)
    log(f"[case] 16-bit accumulator ring lens={lens}")
    qv, q = rand_f16(510, (2, 2, 150, 64))
    kv, k = rand_f16(511, (2, 2, skv, 64))
    vv, v = rand_f16(512, (2, 2, skv, 64))
    out, lse = ops.ring_fwd(q, k, v, len(lens), list(lens), convert_to_fp32=False)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    ro, rl = oracle.ring_attention(qv, kv, vv, lens)
    parity(out, lse, ro, rl, f"fp16 accumulator ring {lens}", FP16_BARS)
