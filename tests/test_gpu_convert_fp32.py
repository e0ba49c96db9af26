"""convert_to_fp32 ("Parallelism" API page, ContextParallelConfig): the default
keeps ring partials and their merges in fp32; False keeps the running output in
the output dtype between chunk steps.  Error study of both against the fp64
oracle over ring degrees 2, 4 and 8, plus edge cases of the 16-bit accumulator."""
import numpy as np
import pytest
import torch

import oracle
from context_attention_diffusion_non_amd import _lib, ops
from tests.gpu_util import BF16_BARS, FP16_BARS, log, parity, rand_bf16, rand_f16, to_np

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


def test_convert_to_fp32_fp32_out_is_identical(study_inputs):
    x = study_inputs
    a = ops.ring_fwd(x["q"], x["k"], x["v"], 4, out_dtype=torch.float32)
    b = ops.ring_fwd(x["q"], x["k"], x["v"], 4, out_dtype=torch.float32, convert_to_fp32=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


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
