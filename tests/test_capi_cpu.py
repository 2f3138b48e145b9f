"""The C-ABI library loads and exports what its header declares (CPU only).

No compute call is made here: only entry points whose host-side validation
rejects the arguments before any HIP call, and pure-host helpers.
"""

import ctypes
import os
import re
import subprocess

import pytest

import ring_attention_chunk_amd as ra
from ring_attention_chunk_amd import api
from ring_attention_chunk_amd.build import LIB, build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attention_chunk.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        build_library()
    return ra.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("ra_attention_chunk_stats", "ra_merge_chunk_stats", "ra_ring_attention"):
        assert n in names
    assert sorted(api.EXPORTS) == names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(ra_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    assert lib.ra_status_string(0) == b"ok"
    assert lib.ra_status_string(6) == b"workspace too small"
    assert lib.ra_status_string(99) == b"unknown status"


def test_workspace_size(lib):
    assert lib.ra_ring_workspace_bytes(1, 8, 64, 4096, 0, 0, 1) % 256 == 0
    assert lib.ra_ring_workspace_bytes(1, 32, 128, 8192, 65536, 64, 2) >= 64 * 64 + 2 * 24
    assert lib.ra_ring_workspace_bytes(1, 32, 128, 8192, 65536, 100, 1) > \
        lib.ra_ring_workspace_bytes(1, 32, 128, 8192, 65536, 10, 1)
    # a grid too small for the chip gets room for per-key-range partials
    small = lib.ra_ring_workspace_bytes(1, 8, 64, 4096, 32768, 8, 1)
    assert small >= 2 * 8 * 4096 * 66 * 4
    assert small % 256 == 0
    big = lib.ra_ring_workspace_bytes(1, 32, 128, 8192, 65536, 8, 1)
    assert big < 1 << 16  # enough query tiles: tables only


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _ring(lib, dtype=1, B=1, Hq=2, Hkv=2, d=64, segs=None, nseg=1, chunks=None, nch=1, causal=0,
          scale=0.125, ws=None, wsb=0, out=FAKE):
    seg = (api.QSegment * 1)(api.QSegment(4, 0)) if segs is None else segs
    ch = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 2 * 8 * 64, 8 * 64, 64)) if chunks is None else chunks
    return lib.ra_ring_attention(dtype, B, Hq, Hkv, d, FAKE, seg, nseg, ch, nch, causal, scale, ws, wsb, out,
                                 None, None)


def test_ring_validation_codes(lib):
    assert _ring(lib, dtype=7) == 3
    assert _ring(lib, Hq=3, Hkv=2) == 2
    assert _ring(lib, d=129) == 4
    assert _ring(lib, d=0) == 4
    assert _ring(lib, nseg=0) == 1
    assert _ring(lib, scale=0.0) == 2
    assert _ring(lib, scale=float("nan")) == 2
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, -1, 0, 0, 0, 64))
    assert _ring(lib, chunks=bad) == 2
    bad = (api.KVChunk * 1)(api.KVChunk(None, FAKE, 8, 0, 0, 0, 64))
    assert _ring(lib, chunks=bad) == 1
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, -3, 0, 0, 64))
    assert _ring(lib, chunks=bad) == 2
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, 32))  # row stride below head_dim
    assert _ring(lib, chunks=bad) == 2
    seg = (api.QSegment * 1)(api.QSegment(4, -1))
    assert _ring(lib, segs=seg, causal=1) == 2
    # position steps: negative is refused; a step that carries the last key past 2^31-2 is refused
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, 64, -2))
    assert _ring(lib, chunks=bad) == 2
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 5, 0, 0, 64, 1 << 29))
    assert _ring(lib, chunks=bad) == 2
    assert b"positions" in lib.ra_last_error()
    seg = (api.QSegment * 1)(api.QSegment(4, 0, -1))
    assert _ring(lib, segs=seg) == 2
    seg = (api.QSegment * 1)(api.QSegment(4, 3, 1 << 30))
    assert _ring(lib, segs=seg, causal=1) == 2
    assert _ring(lib, out=None) == 1
    # the forward kernels keep a chunk's row stride in 32 bits: 2^31 elements or more is refused
    bad = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, 1 << 31))
    assert _ring(lib, chunks=bad) == 4
    assert b"row stride" in lib.ra_last_error()
    ok = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, (1 << 31) - 1))
    assert _ring(lib, chunks=ok) == 6  # accepted; fails later, on the missing workspace
    assert _ring(lib, ws=None, wsb=0) == 6
    assert _ring(lib, ws=ctypes.c_void_p(0x1010), wsb=1 << 20) == 6  # misaligned
    assert b"workspace" in lib.ra_last_error()


def test_noalloc_refuses_a_share_beyond_its_scratch(lib):
    """Host-side check only: a short query share against many keys needs key-range partials beyond the static
    scratch array, and the allocation-free call refuses it before any HIP call."""
    seg = (api.QSegment * 1)(api.QSegment(2048, 0))
    ch = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 1 << 20, 0, 0, 0, 128))
    need = lib.ra_ring_workspace_bytes(1, 8, 128, 2048, 1 << 20, 1, 1)
    assert need > 32 << 20
    st = lib.ra_ring_attention_noalloc(1, 1, 8, 1, 128, FAKE, seg, 1, ch, 1, 0, 0.088, FAKE, None, None)
    assert st == 6
    assert b"static scratch" in lib.ra_last_error()
    # the same validation as the workspace call before that
    assert lib.ra_ring_attention_noalloc(1, 1, 3, 2, 64, FAKE, seg, 1, ch, 1, 0, 0.1, FAKE, None, None) == 2
    assert lib.ra_ring_attention_noalloc(1, 1, 8, 1, 128, FAKE, seg, 1, ch, 1, 0, 0.1, None, None, None) == 1


def test_block_sparse_validation(lib):
    """Host-side checks only: block sizes, mask extent against every position, and the mask pointer."""
    seg = (api.QSegment * 1)(api.QSegment(64, 128))
    ch = (api.KVChunk * 2)(api.KVChunk(FAKE, FAKE, 256, 0, 0, 0, 64), api.KVChunk(FAKE, FAKE, 256, 256, 0, 0, 64))
    need = lib.ra_block_sparse_workspace_bytes(1, 2, 64, 64, 512, 2, 1, 4, 4)
    assert need % 256 == 0 and need > lib.ra_ring_workspace_bytes(1, 2, 64, 64, 512, 2, 1)

    def call(mask=FAKE, nqb=4, nkb=4, bq=128, bk=128, causal=0, ws=None, wsb=0):
        return lib.ra_ring_attention_block_sparse(1, 1, 2, 2, 64, FAKE, seg, 1, ch, 2, causal, 0.125, mask, nqb, nkb,
                                                  bq, bk, ws, wsb, FAKE, None, None)

    assert call(bq=96) == 2  # not a power of two
    assert call(bk=0) == 2
    assert call(nqb=1) == 2  # queries at 128..191 lie in query block 1
    assert b"query segment" in lib.ra_last_error()
    assert call(nkb=3) == 2  # keys reach position 511, key block 3
    assert b"chunk" in lib.ra_last_error()
    assert call(mask=None) == 1
    assert call() == 6  # all valid: fails on the missing workspace
    assert call(ws=ctypes.c_void_p(0x1000), wsb=need - 256) == 6


def test_empty_work_is_a_no_op(lib):
    seg = (api.QSegment * 1)(api.QSegment(0, 0))
    assert _ring(lib, segs=seg) == 0  # no queries: nothing to launch
    assert _ring(lib, B=0) == 0
    assert lib.ra_merge_chunk_stats(0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert lib.ra_last_error() == b""


def test_stats_and_merge_validation(lib):
    ch = api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, 64)
    st = lib.ra_attention_chunk_stats
    assert st(1, 1, 2, 2, 64, FAKE, 4, None, 0.1, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert st(1, 1, 2, 2, 64, FAKE, -1, ctypes.byref(ch), 0.1, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert st(1, 1, 2, 2, 64, FAKE, 4, ctypes.byref(ch), 0.1, None, FAKE, FAKE, None, 0, None) == 1
    assert st(2, 1, 2, 2, 64, FAKE, 4, ctypes.byref(ch), 0.1, FAKE, FAKE, FAKE, None, 0, None) == 3
    wide = api.KVChunk(FAKE, FAKE, 8, 0, 0, 0, 1 << 32)
    assert st(1, 1, 2, 2, 64, FAKE, 4, ctypes.byref(wide), 0.1, FAKE, FAKE, FAKE, None, 0, None) == 4
    assert st(1, 1, 2, 2, 64, FAKE, 4, ctypes.byref(ch), 0.1, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1010), 1 << 20,
              None) == 6  # misaligned workspace
    # a short query share against a long chunk gets room for key-range partials; a large one none
    assert lib.ra_chunk_stats_workspace_bytes(1, 8, 64, 1024, 4096) >= 2 * 8 * 1024 * 66 * 4
    assert lib.ra_chunk_stats_workspace_bytes(1, 8, 64, 4096, 4096) == 0  # one workgroup per CU already
    assert lib.ra_merge_chunk_stats(-1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.ra_merge_chunk_stats(5, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.ra_merge_chunk_stats(5, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1


def test_python_layer_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ra.RingAttentionError):
        ra.ring_attention(q, [q], [q])
    with pytest.raises(ra.RingAttentionError):
        ra.attention_chunk_stats(q, q, q)


def test_kernel_timer_read_rejects_null(lib):
    # host-side check only: no event is created or read
    assert lib.ra_kernel_timer_read(None, None) == 1


def test_backward_validation_codes(lib):
    seg = (api.QSegment * 1)(api.QSegment(4, 0))
    ch = (api.KVChunk * 1)(api.KVChunk(FAKE, FAKE, 8, 0, 2 * 8 * 64, 8 * 64, 64))

    def bwd(dtype=1, d=64, Hq=2, Hkv=2, ws=None, wsb=0, dq=FAKE):
        return lib.ra_ring_attention_backward(dtype, 1, Hq, Hkv, d, FAKE, seg, 1, ch, 1, 0, 0.125, FAKE, FAKE, FAKE,
                                              ws, wsb, dq, FAKE, FAKE, None)

    assert bwd(dtype=0) == 4  # fp32: not supported by the backward kernels
    assert bwd(d=36) == 4  # not a multiple of 8
    assert bwd(Hq=3) == 2
    assert bwd(dq=None) == 1
    assert bwd() == 6  # no workspace
    assert b"workspace" in lib.ra_last_error()
    need = lib.ra_ring_backward_workspace_bytes(1, 2, 64, 4, 8, 1, 1)
    assert need % 256 == 0 and need >= 4 * (4 + 8) + 4 * 2 * 4
    # a short share with many keys gets room for partial dq of several key ranges
    small = lib.ra_ring_backward_workspace_bytes(1, 8, 64, 4096, 32768, 8, 1)
    assert small >= 2 * 8 * 4096 * 64 * 4
    big = lib.ra_ring_backward_workspace_bytes(1, 32, 128, 8192, 65536, 8, 2)
    assert big < 32 * 8192 * 128 * 4  # enough query rows: no partials
