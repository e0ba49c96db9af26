"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU.  Every call here
fails validation (or is pure host code), so nothing is launched."""
import ctypes

import pytest

from context_attention_diffusion_non_amd import _lib

FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000000)
FAKE3 = ctypes.c_void_p(0x40000000)
FAKE4 = ctypes.c_void_p(0x60000000)
FAKE5 = ctypes.c_void_p(0x70000000)
NULL = ctypes.c_void_p(0)
OK, ERR_NULL, ERR_SHAPE, ERR_DEGREE, ERR_INDIV, ERR_CHUNKS, ERR_DTYPE, ERR_WS, ERR_ALIAS = range(9)


@pytest.fixture(scope="module")
def L(lib_path):
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _lib.declared_functions()
    assert {"cpattn_block_fwd", "cpattn_lse_merge", "cpattn_ring_fwd", "cpattn_ulysses_permute",
            "cpattn_ring_fwd_workspace_bytes", "cpattn_status_string", "cpattn_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in cpattn.h but not exported"


def test_version_and_strings(L):
    assert L.cpattn_version() >= 100
    for s in range(10):
        assert L.cpattn_status_string(s)
    assert L.cpattn_status_string(99) == b"unknown status"


def block(L, q=FAKE, k=FAKE2, v=FAKE3, out=FAKE4, lse=FAKE5, B=1, H=2, Sq=16, Skv=16, ld=16, d=128, idt=0, odt=1):
    return L.cpattn_block_fwd(q, k, v, out, lse, B, H, Sq, Skv, ld, d, 0.0, idt, odt, NULL)


def test_block_fwd_validation(L):
    assert block(L, B=0) == ERR_SHAPE
    assert block(L, H=-1) == ERR_SHAPE
    assert block(L, Sq=-1) == ERR_SHAPE
    assert block(L, Skv=32, ld=16) == ERR_SHAPE
    assert block(L, d=96) == ERR_SHAPE
    assert b"64 or 128" in L.cpattn_last_error()
    assert block(L, idt=7) == ERR_DTYPE
    assert block(L, odt=3) == ERR_DTYPE
    assert block(L, idt=-1) == ERR_DTYPE
    assert block(L, q=NULL) == ERR_NULL
    assert block(L, k=NULL) == ERR_NULL
    assert block(L, lse=NULL) == ERR_NULL
    assert block(L, out=FAKE) == ERR_ALIAS           # out == q
    assert block(L, lse=FAKE2) == ERR_ALIAS          # lse == k
    assert block(L, B=1 << 40, H=1 << 40) == ERR_SHAPE
    # empty query shard is a no-op even with NULL pointers
    assert block(L, q=NULL, out=NULL, lse=NULL, Sq=0) == OK


def ring(L, degree=2, lens=None, Skv=16, ws=NULL, ws_bytes=0, odt=1, B=1, H=2, Sq=16, d=128):
    arr = None if lens is None else (ctypes.c_int64 * len(lens))(*lens)
    return L.cpattn_ring_fwd(FAKE, FAKE2, FAKE3, FAKE4, FAKE5, B, H, Sq, Skv, d, 0.0, degree, arr, ws, ws_bytes,
                             0, odt, NULL)


def test_ring_fwd_validation(L):
    assert ring(L, degree=0) == ERR_DEGREE
    assert ring(L, degree=-3) == ERR_DEGREE
    assert ring(L, degree=3, Skv=16) == ERR_INDIV      # plain ring needs S % N == 0
    assert b"not divisible" in L.cpattn_last_error()
    assert ring(L, degree=3, lens=[6, 6, 5], Skv=16) == ERR_CHUNKS
    assert ring(L, degree=3, lens=[6, 11, -1], Skv=16) == ERR_CHUNKS
    # lengths whose int64 sum wraps around to exactly Skv are rejected, not summed
    big = (1 << 63) - 1
    assert ring(L, degree=3, lens=[big, big, 18], Skv=16) == ERR_CHUNKS
    assert ring(L, degree=3, lens=[16, big, big], Skv=16) == ERR_CHUNKS
    # 513 planes of one 16-row query tile (more than a round of 512 four-wave workgroups) against
    # 16 key tiles: two rounds of 256 eight-wave workgroups, then the leftover tile's 16 tiles
    # split over the other 255 (no head: round(16 / 256) = 0), so the step writes pieces:
    # 2 slots x 256 ranges x 16 rows of d fp32 values, then their LSE.  Any output dtype.
    for odt in (0, 1, 2):
        assert ring(L, degree=2, odt=odt, H=513, Skv=1024) == ERR_WS
    need = 2 * 256 * 16 * 128 * 4 + 2 * 256 * 16 * 4
    assert L.cpattn_ring_fwd_workspace_bytes(1, 513, 16, 128, 2, 0) == need
    big_ws = ctypes.c_void_p(0x50000000)
    assert ring(L, degree=2, H=513, Skv=1024, ws=big_ws, ws_bytes=need - 1) == ERR_WS
    assert ring(L, degree=2, H=513, Skv=1024, ws=ctypes.c_void_p(0x50000010), ws_bytes=need) == ERR_WS  # alignment
    assert ring(L, degree=2, H=513, Skv=1024, ws=FAKE4, ws_bytes=need) == ERR_ALIAS                    # ws == out
    # more chunks than one launch takes: the per-chunk loop and its fp32 accumulator
    lens = [8] * 130
    assert ring(L, degree=130, lens=lens, Skv=1040, odt=0) == ERR_WS


def test_workspace_bytes(L):
    """The one-launch ring step's most: two slots per range (256 eight-wave ranges at d = 128,
    512 at d = 64) of min(256, Sq) rows x d fp32 values, then their LSE at a 256-byte offset --
    whatever the chunking and output dtype.  Past 128 chunks: the per-chunk loop's fp32
    accumulator, none for fp32 output."""
    f = L.cpattn_ring_fwd_workspace_bytes
    slots = lambda ranges, rows, d: 2 * ranges * rows * d * 4 + 2 * ranges * rows * 4
    assert f(1, 24, 2304, 128, 2, 0) == slots(256, 256, 128)
    assert f(1, 24, 2304, 128, 1, 0) == slots(256, 256, 128)
    assert f(1, 24, 2304, 128, 4, 1) == slots(256, 256, 128)
    assert f(2, 24, 4096, 64, 2, 2) == slots(512, 256, 64)
    assert f(1, 2, 16, 128, 2, 0) == slots(256, 16, 128)
    assert f(1, 2, 0, 128, 2, 0) == 0
    assert f(1, 24, 2304, 128, 200, 0) == 24 * 2304 * 128 * 4
    assert f(1, 24, 2304, 128, 200, 1) == 0
    assert f(0, 24, 2304, 128, 2, 0) == 0


def perm(L, inp=FAKE, out=FAKE2, B=1, S_loc=8, H=4, d=64, P=2, g=0, direction=0, eb=2):
    return L.cpattn_ulysses_permute(inp, out, B, S_loc, H, d, P, g, direction, eb, NULL)


def test_permute_validation(L):
    assert perm(L, P=0) == ERR_DEGREE
    assert perm(L, g=2) == ERR_DEGREE
    assert perm(L, g=-2) == ERR_DEGREE
    assert perm(L, H=6, P=4) == ERR_INDIV
    assert perm(L, direction=2) == ERR_DTYPE
    assert perm(L, eb=3) == ERR_DTYPE
    assert perm(L, inp=NULL) == ERR_NULL
    assert perm(L, out=ctypes.c_void_p(0x10000 + 64)) == ERR_ALIAS
    assert perm(L, S_loc=0) == OK


def test_merge_validation(L):
    m = L.cpattn_lse_merge
    assert m(FAKE, FAKE2, FAKE3, FAKE4, -1, 128, 1, NULL) == ERR_SHAPE
    assert m(FAKE, FAKE2, FAKE3, FAKE4, 10, 96, 1, NULL) == ERR_SHAPE
    assert m(FAKE, FAKE2, FAKE3, FAKE4, 10, 128, 5, NULL) == ERR_DTYPE
    assert m(FAKE, NULL, FAKE3, FAKE4, 10, 128, 1, NULL) == ERR_NULL
    assert m(FAKE, FAKE2, FAKE, FAKE4, 10, 128, 1, NULL) == ERR_ALIAS
    assert m(FAKE, FAKE2, FAKE3, FAKE4, 0, 128, 1, NULL) == OK


def test_python_binding_refuses_cpu_tensors(lib_path):
    import torch
    from context_attention_diffusion_non_amd import ops
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.ring_fwd(q, q, q, 1)


@pytest.mark.parametrize("fn", ["block_fwd", "ring_fwd", "unified_fwd"])
def test_python_binding_refuses_mixed_dtypes(fn, monkeypatch):
    """k/v are read at q's element size, so a dtype mismatch must raise before any library call."""
    import torch
    from context_attention_diffusion_non_amd import ops

    def no_call():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(_lib, "lib", no_call)
    if fn == "unified_fwd":
        q = torch.zeros(2, 1, 4, 2, 64, dtype=torch.float32)
        kv = torch.zeros(2, 1, 4, 2, 64, dtype=torch.bfloat16)
        call = lambda a, b, c: ops.unified_fwd(a, b, c, 2, 1, 0, 0)
    else:
        q = torch.zeros(1, 1, 4, 64, dtype=torch.float32)
        kv = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
        call = (lambda a, b, c: ops.block_fwd(a, b, c)) if fn == "block_fwd" else \
            (lambda a, b, c: ops.ring_fwd(a, b, c, 1))
    with pytest.raises(TypeError, match="share one dtype"):
        call(q, kv, kv)
    with pytest.raises(TypeError, match="share one dtype"):
        call(q, q, kv)
    with pytest.raises(TypeError, match="share one dtype"):
        call(kv, kv, q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def unified(L, q=FAKE, k=FAKE2, v=FAKE3, out=FAKE4, lse=FAKE5, B=1, S_loc=8, H=4, d=64, R=2, U=2, rr=0, ur=0,
            ws=NULL, ws_bytes=0, idt=0, odt=0):
    return L.cpattn_unified_fwd(q, k, v, out, lse, B, S_loc, H, d, 0.0, R, U, rr, ur, ws, ws_bytes, idt, odt, NULL)


def test_unified_validation(L):
    assert unified(L, R=0) == ERR_DEGREE
    assert unified(L, U=0) == ERR_DEGREE
    assert unified(L, R=300, U=300) == ERR_DEGREE          # grid larger than a launch dimension allows
    assert unified(L, rr=2) == ERR_DEGREE
    assert unified(L, ur=-1) == ERR_DEGREE
    assert unified(L, H=6, U=4) == ERR_INDIV
    assert unified(L, d=96) == ERR_SHAPE
    assert unified(L, idt=7) == ERR_DTYPE
    assert unified(L, q=NULL, ws=ctypes.c_void_p(0x70000000), ws_bytes=1 << 20) == ERR_NULL
    assert unified(L) == ERR_WS                               # no workspace
    need = L.cpattn_unified_fwd_workspace_bytes(1, 8, 4, 64, 2, 2, 0, 0)
    assert unified(L, ws=ctypes.c_void_p(0x70000000), ws_bytes=need - 1) == ERR_WS
    assert unified(L, ws=ctypes.c_void_p(0x70000010), ws_bytes=need) == ERR_WS  # alignment
    assert unified(L, ws=FAKE, ws_bytes=need) == ERR_ALIAS                      # workspace over q
    assert unified(L, S_loc=0) == OK


def test_unified_workspace_bytes(L):
    f = L.cpattn_unified_fwd_workspace_bytes
    B, S_loc, H, d, R, U = 2, 1024, 24, 64, 2, 2
    hq, seg, allk = H // U, U * S_loc, R * U * S_loc
    q_b, kv_b = B * hq * seg * d * 2, B * hq * allk * d * 2
    ring_b = 2 * 512 * 256 * d * 4 + 2 * 512 * 256 * 4       # the ring step's slots at d = 64
    assert f(B, S_loc, H, d, R, U, 2, 2) == q_b + 2 * kv_b + ring_b
    assert f(B, S_loc, H, d, R, U, 2, 1) == q_b + 2 * kv_b + ring_b
    assert f(B, S_loc, H, d, 1, U, 0, 0) == q_b + 2 * (B * hq * seg * d * 2) + ring_b   # one ring segment
    assert f(B, S_loc, 25, d, R, U, 0, 0) == 0                          # H % U != 0


def anyperm(L, inp=FAKE, out=FAKE2, B=1, H=5, d=64, P=2, sl=(3, 2), hl=(3, 2), g=0, direction=0, eb=2):
    a = None if sl is None else (ctypes.c_int64 * len(sl))(*sl)
    b = None if hl is None else (ctypes.c_int64 * len(hl))(*hl)
    return L.cpattn_ulysses_anything_permute(inp, out, B, H, d, P, a, b, g, direction, eb, NULL)


def test_anything_permute_validation(L):
    assert anyperm(L, P=0, sl=(), hl=()) == ERR_DEGREE
    assert anyperm(L, P=33, sl=(1,) * 33, hl=(1,) * 33, H=33) == ERR_DEGREE
    assert anyperm(L, g=2) == ERR_DEGREE
    assert anyperm(L, sl=None) == ERR_NULL
    assert anyperm(L, hl=(3, 1)) == ERR_CHUNKS          # head counts must sum to H
    assert anyperm(L, sl=(3, -1)) == ERR_CHUNKS
    assert anyperm(L, direction=3) == ERR_DTYPE
    assert anyperm(L, eb=3) == ERR_DTYPE
    assert anyperm(L, inp=NULL) == ERR_NULL
    assert anyperm(L, out=ctypes.c_void_p(0x10000 + 128)) == ERR_ALIAS
    assert anyperm(L, sl=(0, 0)) == OK                    # no tokens: nothing to do
    assert anyperm(L, out=NULL, H=5, hl=(5, 0), g=1) == OK  # a group without heads: nothing to write


def test_ring_fwd_cfg_needs_no_workspace_without_fp32(L):
    f = L.cpattn_ring_fwd_cfg
    # bf16 out, 2 chunks, split query tiles: the fp32 default needs the pieces' workspace,
    # convert_to_fp32=0 (one launch per chunk, the output as the running accumulator) does not
    assert f(FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 513, 16, 1024, 128, 0.0, 2, None, 1, NULL, 0, 0, 0, NULL) == ERR_WS
    assert f(FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 2, 0, 16, 128, 0.0, 2, None, 0, NULL, 0, 0, 0, NULL) == OK
    assert f(FAKE, FAKE2, FAKE3, FAKE4, FAKE5, 1, 2, 16, 16, 128, 0.0, 0, None, 0, NULL, 0, 0, 0, NULL) == ERR_DEGREE
