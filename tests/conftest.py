import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU oracle time)")


@pytest.fixture(scope="session")
def lib_path():
    """Path of the built C-ABI library; builds it once if nothing is built."""
    from context_attention_diffusion_non_amd import _lib
    path = _lib.library_path()
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build()
    assert os.path.exists(path), f"libcpattn.so was not built at {path}"
    return path


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def pages_example():
    """The pages' correctness shape (ParaAttention README, unified attention
    example): fp16 [B=2, H=24, S=4096, D=64] q/k/v and the unsplit oracle
    attention over all of it (about 10 s of fp64 BLAS, computed once)."""
    import oracle
    from tests.gpu_util import log, rand_f16
    B, H, S, D = 2, 24, 4096, 64
    qv, q = rand_f16(0, (B, H, S, D))
    kv, k = rand_f16(1, (B, H, S, D))
    vv, v = rand_f16(2, (B, H, S, D))
    log("[info] pages example: computing the unsplit oracle")
    ro, rl = oracle.attention(qv, kv, vv)
    return dict(q=q, k=k, v=v, ref_out=ro, ref_lse=rl, S=S)
