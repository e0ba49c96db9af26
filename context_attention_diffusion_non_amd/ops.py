"""Python binding of the cpattn C ABI: torch tensors in, library calls out.

Only argument marshalling happens here: torch provides device memory and the
current HIP stream; every step of the computation runs in the library's
kernels.  The names mirror the C entry points (cpattn_<name>).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import BF16, FP16, FP32, CpattnError, check

_DT = {torch.bfloat16: BF16, torch.float32: FP32, torch.float16: FP16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; cpattn takes bfloat16, float16 or float32")
    return _DT[t.dtype]


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("cpattn tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("cpattn tensors must be contiguous")


def _same_kind(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
    """The library reads k and v at q's element size: all three must share dtype and device."""
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError(f"q, k and v must share one dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    if k.device != q.device or v.device != q.device:
        raise ValueError(f"q, k and v must be on one device (got {q.device}, {k.device}, {v.device})")


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _scale(scale: Optional[float]) -> float:
    return 0.0 if scale is None else float(scale)


def _shape(t: torch.Tensor, shape, name: str) -> None:
    """The library takes raw pointers: every buffer is checked against the sizes it is given."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def block_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, kv_len: Optional[int] = None,
              scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """cpattn_block_fwd: attention of q [B,H,Sq,d] against k/v [B,H,kv_ld,d] rows [0, kv_len)."""
    _same_kind(q, k, v)
    _dev(q, k, v)
    B, H, Sq, d = q.shape
    kv_ld = k.shape[2]
    _shape(k, (B, H, kv_ld, d), "k")
    _shape(v, (B, H, kv_ld, d), "v")
    skv = kv_ld if kv_len is None else int(kv_len)
    if not 0 <= skv <= kv_ld:
        raise ValueError(f"kv_len must lie in [0, {kv_ld}]")
    od = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _dev(out, lse)
    _shape(out, (B, H, Sq, d), "out")
    _shape(lse, (B, H, Sq), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    check(_lib.lib().cpattn_block_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, skv, kv_ld, d,
                                      _scale(scale), _dtype_code(q), _dtype_code(out), _stream(q)))
    return out, lse


def lse_merge(acc_out: torch.Tensor, acc_lse: torch.Tensor, blk_out: torch.Tensor, blk_lse: torch.Tensor) -> None:
    """cpattn_lse_merge: fold (blk_out, blk_lse) into fp32 (acc_out, acc_lse) in place."""
    _dev(acc_out, acc_lse, blk_out, blk_lse)
    if acc_out.dtype != torch.float32 or acc_lse.dtype != torch.float32 or blk_lse.dtype != torch.float32:
        raise TypeError("accumulator and LSE tensors must be float32")
    d = acc_out.shape[-1]
    rows = acc_out.numel() // d if d else 0
    _shape(blk_out, acc_out.shape, "blk_out")
    if acc_lse.numel() != rows or blk_lse.numel() != rows:
        raise ValueError(f"acc_lse and blk_lse must hold {rows} values")
    check(_lib.lib().cpattn_lse_merge(_ptr(acc_out), _ptr(acc_lse), _ptr(blk_out), _ptr(blk_lse), rows, d,
                                      _dtype_code(blk_out), _stream(acc_out)))


def ring_fwd_workspace_bytes(B: int, H: int, Sq: int, d: int, ring_degree: int, out_dtype: torch.dtype) -> int:
    return int(_lib.lib().cpattn_ring_fwd_workspace_bytes(B, H, Sq, d, ring_degree, _DT[out_dtype]))


def ring_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ring_degree: int,
             chunk_lens: Optional[Sequence[int]] = None, *, scale: Optional[float] = None,
             out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             convert_to_fp32: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """cpattn_ring_fwd: q [B,H,Sq,d] against k/v [B,H,Skv,d] split into ring_degree chunks.

    convert_to_fp32=False calls cpattn_ring_fwd_cfg and keeps the running output in the
    output dtype between chunk steps (no workspace)."""
    _same_kind(q, k, v)
    _dev(q, k, v)
    B, H, Sq, d = q.shape
    skv = k.shape[2]
    _shape(k, (B, H, skv, d), "k")
    _shape(v, (B, H, skv, d), "v")
    od = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _dev(out, lse)
    _shape(out, (B, H, Sq, d), "out")
    _shape(lse, (B, H, Sq), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    need = int(_lib.lib().cpattn_ring_fwd_workspace_bytes(B, H, Sq, d, ring_degree, _dtype_code(out)))
    if not convert_to_fp32:
        need = 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lens = None
    if chunk_lens is not None:
        lens = (ctypes.c_int64 * len(chunk_lens))(*[int(x) for x in chunk_lens])
        if len(chunk_lens) != ring_degree:
            raise ValueError("len(chunk_lens) must equal ring_degree")
    if convert_to_fp32:
        st = _lib.lib().cpattn_ring_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, skv, d,
                                        _scale(scale), int(ring_degree), lens, _ptr(workspace), ws_bytes,
                                        _dtype_code(q), _dtype_code(out), _stream(q))
    else:
        st = _lib.lib().cpattn_ring_fwd_cfg(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, skv, d,
                                            _scale(scale), int(ring_degree), lens, 0, _ptr(workspace), ws_bytes,
                                            _dtype_code(q), _dtype_code(out), _stream(q))
    check(st)
    return out, lse


def ring_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ring_degree: int,
                     chunk_lens: Optional[Sequence[int]] = None, *, scale: Optional[float] = None,
                     out: torch.Tensor, lse: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """cpattn_ring_fwd_noalloc: cpattn_ring_fwd on the library's own scratch, no workspace.

    ``out`` and ``lse`` are required (nothing is allocated here either); out's dtype selects
    the output dtype.  Calls that overlap on one GPU share that scratch and must be serialised."""
    _same_kind(q, k, v)
    _dev(q, k, v, out, lse)
    B, H, Sq, d = q.shape
    skv = k.shape[2]
    _shape(k, (B, H, skv, d), "k")
    _shape(v, (B, H, skv, d), "v")
    _shape(out, (B, H, Sq, d), "out")
    _shape(lse, (B, H, Sq), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    lens = None
    if chunk_lens is not None:
        if len(chunk_lens) != ring_degree:
            raise ValueError("len(chunk_lens) must equal ring_degree")
        lens = (ctypes.c_int64 * len(chunk_lens))(*[int(x) for x in chunk_lens])
    check(_lib.lib().cpattn_ring_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, skv, d,
                                             _scale(scale), int(ring_degree), lens, _dtype_code(q),
                                             _dtype_code(out), _stream(q)))
    return out, lse


def ulysses_permute(x: torch.Tensor, degree: int, group: int = 0, direction: int = 0,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cpattn_ulysses_permute.

    direction 0: x [P, B, S_local, H, d] -> [B, H/P, P*S_local, d] (group >= 0) or
                 [P, B, H/P, P*S_local, d] (group == -1).
    direction 1: x [B, H/P, S, d] (or [P, B, H/P, S, d] for group -1) -> ``out``
                 [P, B, S/P, H, d], writing only the group's heads (``out`` must be
                 given, or a zero tensor is created).
    """
    _dev(x)
    eb = x.element_size()
    if direction == 0:
        P, B, S_loc, H, d = x.shape
        if P != degree:
            raise ValueError("x.shape[0] must equal degree")
        hp = H // degree if degree > 0 else 0
        shape = (B, hp, P * S_loc, d) if group >= 0 else (degree, B, hp, P * S_loc, d)
        if out is None:
            out = torch.empty(shape, dtype=x.dtype, device=x.device)
    else:
        if group >= 0:
            B, hp, S, d = x.shape
        else:
            G, B, hp, S, d = x.shape
            if G != degree:
                raise ValueError("x.shape[0] must equal degree for group -1")
        if degree < 1 or S % degree:
            raise ValueError("S must divide by degree")
        S_loc, H = S // degree, hp * degree
        shape = (degree, B, S_loc, H, d)
        if out is None:
            out = torch.zeros(shape, dtype=x.dtype, device=x.device)
    _dev(out)
    _shape(out, shape, "out")
    if out.dtype != x.dtype:
        raise TypeError("out must have x's dtype")
    check(_lib.lib().cpattn_ulysses_permute(_ptr(x), _ptr(out), B, S_loc, H, d, int(degree), int(group),
                                            int(direction), eb, _stream(x)))
    return out


def even_split(n: int, parts: int):
    """Default Ulysses Anything split: the first n mod parts pieces one longer."""
    base, extra = divmod(int(n), int(parts))
    return [base + (1 if i < extra else 0) for i in range(parts)]


def ulysses_anything_permute(x: torch.Tensor, B: int, H: int, d: int, seq_lens: Sequence[int],
                             head_lens: Optional[Sequence[int]] = None, group: int = 0, direction: int = 0,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cpattn_ulysses_anything_permute.

    direction 0: x = the packed sequence shards (shard r = [B, seq_lens[r], H, d] back to back,
                 B*S*H*d elements) -> [B, head_lens[group], S, d] (group >= 0) or every group
                 packed back to back as a flat tensor (group == -1).
    direction 1: the inverse; ``out`` holds the packed shards (created as zeros if not given).
    head_lens defaults to ``even_split(H, len(seq_lens))``.
    """
    _dev(x)
    P = len(seq_lens)
    if head_lens is None:
        head_lens = even_split(H, P)
    if len(head_lens) != P:
        raise ValueError("head_lens needs one entry per shard")
    S = int(sum(seq_lens))
    seq_numel = B * S * H * d
    head_numel = seq_numel if group < 0 else B * int(head_lens[group]) * S * d
    if direction == 0:
        if x.numel() != seq_numel:
            raise ValueError(f"x must hold the packed shards ({seq_numel} elements)")
        if out is None:
            shape = (B, int(head_lens[group]), S, d) if group >= 0 else (head_numel,)
            out = torch.empty(shape, dtype=x.dtype, device=x.device)
        want = head_numel
    else:
        if x.numel() != head_numel:
            raise ValueError(f"x must hold {head_numel} elements")
        if out is None:
            out = torch.zeros(seq_numel, dtype=x.dtype, device=x.device)
        want = seq_numel
    _dev(out)
    if out.numel() != want or out.dtype != x.dtype:
        raise ValueError(f"out must hold {want} elements of x's dtype")
    sl = (ctypes.c_int64 * P)(*[int(n) for n in seq_lens])
    hl = (ctypes.c_int64 * P)(*[int(n) for n in head_lens])
    check(_lib.lib().cpattn_ulysses_anything_permute(_ptr(x), _ptr(out), B, H, d, P, sl, hl, int(group),
                                                     int(direction), x.element_size(), _stream(x)))
    return out


def unified_fwd_workspace_bytes(B: int, S_local: int, H: int, d: int, ring_degree: int, ulysses_degree: int,
                                in_dtype: torch.dtype, out_dtype: torch.dtype) -> int:
    return int(_lib.lib().cpattn_unified_fwd_workspace_bytes(B, S_local, H, d, ring_degree, ulysses_degree,
                                                              _DT[in_dtype], _DT[out_dtype]))


def unified_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ring_degree: int, ulysses_degree: int,
                ring_rank: int, ulysses_rank: int, *, scale: Optional[float] = None,
                out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """cpattn_unified_fwd: rank (ring_rank, ulysses_rank)'s share of Unified attention.

    q, k, v: [W, B, S_local, H, d] sequence shards of all W = ring_degree * ulysses_degree ranks.
    Returns out [B, H/U, U*S_local, d] and lse [B, H/U, U*S_local] (head-sharded, before the
    reverse regroup, which is ``ulysses_permute(..., direction=1)`` over a Ulysses group's outputs).
    """
    _same_kind(q, k, v)
    _dev(q, k, v)
    W, B, S_loc, H, d = q.shape
    _shape(k, q.shape, "k")
    _shape(v, q.shape, "v")
    if ring_degree < 1 or ulysses_degree < 1 or W != ring_degree * ulysses_degree:
        raise ValueError("q.shape[0] must equal ring_degree * ulysses_degree")
    if H % ulysses_degree:
        raise ValueError("H must divide by ulysses_degree")
    hq, seg = H // ulysses_degree, ulysses_degree * S_loc
    od = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, hq, seg, d), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((B, hq, seg), dtype=torch.float32, device=q.device)
    _dev(out, lse)
    _shape(out, (B, hq, seg, d), "out")
    _shape(lse, (B, hq, seg), "lse")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    need = int(_lib.lib().cpattn_unified_fwd_workspace_bytes(B, S_loc, H, d, ring_degree, ulysses_degree,
                                                              _dtype_code(q), _dtype_code(out)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(_lib.lib().cpattn_unified_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, S_loc, H, d,
                                        _scale(scale), int(ring_degree), int(ulysses_degree), int(ring_rank),
                                        int(ulysses_rank), _ptr(workspace), ws_bytes, _dtype_code(q),
                                        _dtype_code(out), _stream(q)))
    return out, lse


__all__ = ["block_fwd", "lse_merge", "ring_fwd", "ring_fwd_workspace_bytes", "ring_fwd_noalloc", "ulysses_permute",
           "unified_fwd",
           "ulysses_anything_permute", "even_split",
           "unified_fwd_workspace_bytes", "CpattnError", "BF16", "FP16", "FP32"]
