"""cpattn: per-rank context-parallel attention for AMD MI355X (gfx950).

The computation a ring / Ulysses context-parallel rank runs inside its
attention backend -- attention of a query shard against K/V chunks, each chunk
emitting a partial output and its log-sum-exp, partials merged in fp32 by LSE
rescaling, and the Ulysses sequence<->head regroup -- as hand-written HIP
kernels behind a C ABI (include/cpattn.h).  This package is the thin Python
binding: torch supplies device memory and streams, the library computes.
"""
from ._lib import CpattnError, library_path  # noqa: F401


def __getattr__(name):
    # the torch-facing ops load lazily so that importing the package (e.g. for
    # the workload generator) does not need torch or the built library
    if name in ("block_fwd", "lse_merge", "ring_fwd", "ring_fwd_workspace_bytes", "ulysses_permute"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
