"""Host-only checks of the C interface: the library loads, exports every
function include/minf.h declares, and argument validation answers with the
documented status codes before anything reaches a GPU (no device pointer is
ever dereferenced by these calls)."""
import ctypes
import os
import re

import pytest

import long_context_prefill_amd as M
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from long_context_prefill_amd import build
        build.build()
    return M.load_library()


def _declared():
    txt = open(os.path.join(ROOT, "include", "minf.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(minf_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(M.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.minf_version().decode().startswith("minf")


def test_struct_layouts_match_header():
    assert ctypes.sizeof(M.MinfProblem) == 40
    assert ctypes.sizeof(M.MinfHeadCfg) == 32
    assert ctypes.sizeof(M.MinfSizes) == 64
    assert ctypes.sizeof(M.MinfTiles) == 120


def _prob(**kw):
    base = dict(B=1, Hq=4, Hkv=2, n=1000, dh=128, in_dtype="bf16", out_dtype="f32")
    base.update(kw)
    return M.make_problem(**base)


HEADS = [gen.ashape(16, 100), gen.vslash(64, 40, 60), gen.bsparse(4), gen.vslash(32, 1000, 2000)]


def test_query_sizes(lib):
    s = M.minf_query_sizes(_prob(), M.make_heads(HEADS))
    assert s.nq == 16
    assert s.max_v == 1024          # min(1000, n) rounded up to 32
    assert s.max_s == 1000          # min(2000, n)
    assert s.max_kb == 4
    assert s.max_chunks == (1000 + 63 + 31) // 32 + 1000 + 1
    assert s.ws_bytes > 0
    assert s.bits_words == 0        # only for exact slash pairs
    # span tails: at most 31 offsets per range and at most n + 63 offsets in
    # all, in whole packed chunks of 32
    assert s.max_tail == 1088       # min(31 * 1000, 1000 + 63) rounded up to 32


def test_query_sizes_exact_slash_pairs(lib):
    """slash_tile=1 (Eq. 5 pairs) sizes the two per-head bitmaps: offset d
    at bit n + 127 - d, column j at bit j + 128, 32-bit words, with room for
    the three-word windows the attention reads."""
    s = M.minf_query_sizes(_prob(slash_tile=1), M.make_heads(HEADS))
    assert s.bits_words == (1000 + 2 * 128 + 64 + 31) // 32 + 2
    assert s.bits_words * 32 >= 1000 + 128 + 128 + 64
    # no Vertical-Slash head: no bitmaps
    s = M.minf_query_sizes(_prob(slash_tile=1), M.make_heads([gen.ashape(4, 8)] * 4))
    assert s.bits_words == 0


@pytest.mark.parametrize("kw,heads,status", [
    (dict(Hq=3, Hkv=2), HEADS[:3], M.MINF_EINVAL),
    (dict(dh=96), HEADS, M.MINF_EUNSUPPORTED),
    (dict(n=0), HEADS, M.MINF_EINVAL),
    (dict(block=32), HEADS, M.MINF_EUNSUPPORTED),
    (dict(slash_tile=16), HEADS, M.MINF_EINVAL),
    (dict(scale=-1.0), HEADS, M.MINF_EINVAL),
    (dict(), [gen.ashape(-1, 3)] + HEADS[1:], M.MINF_EINVAL),
    (dict(), [gen.vslash(65, 1, 1)] + HEADS[1:], M.MINF_EUNSUPPORTED),
    (dict(), [gen.vslash(0, 1, 1)] + HEADS[1:], M.MINF_EINVAL),
    (dict(), [gen.bsparse(0)] + HEADS[1:], M.MINF_EINVAL),
    (dict(), [gen.bsparse(2, 8)] + HEADS[1:], M.MINF_EINVAL),
    (dict(), [gen.HeadCfg(7)] + HEADS[1:], M.MINF_EINVAL),
    # a Block-Sparse row of more than 32768 key blocks (n > 2^21) is refused
    (dict(n=(1 << 21) + 1, Hq=4, Hkv=1), HEADS, M.MINF_EUNSUPPORTED),
])
def test_validation_errors(lib, kw, heads, status):
    p = _prob(**kw)
    with pytest.raises(M.MinfError) as e:
        M.minf_query_sizes(p, M.make_heads(heads))
    assert e.value.status == status
    assert lib.minf_last_error().decode()


def test_calls_reject_before_launch(lib):
    """Null buffers and short workspaces are refused synchronously; the fake
    pointers below are never dereferenced because validation fails first."""
    p = _prob()
    h = M.make_heads(HEADS)
    fake = 0x1000
    ts = M.MinfTiles()
    st = lib.minf_vs_index(ctypes.byref(p), h, None, fake, fake, fake, None, None, fake, 1 << 40, None)
    assert st == M.MINF_EINVAL
    st = lib.minf_vs_index(ctypes.byref(p), h, fake, fake, fake, fake, None, None, fake, 16, None)
    assert st == M.MINF_EWORKSPACE
    st = lib.minf_bs_index(ctypes.byref(p), h, fake, fake, None, fake, fake, 1 << 40, None)
    assert st == M.MINF_EINVAL
    # the single-launch proxy needs its status word
    st = lib.minf_vs_index_fused(ctypes.byref(p), h, fake, fake, fake, fake, None, None, fake, 1 << 40, None, None)
    assert st == M.MINF_EINVAL and "status" in lib.minf_last_error().decode()
    st = lib.minf_build_tiles(ctypes.byref(p), h, fake, fake, fake, fake, ctypes.byref(ts), fake, 1 << 40, None)
    assert st == M.MINF_EINVAL          # tiles has no kept_edges / status
    st = lib.minf_sparse_attn(ctypes.byref(p), h, fake, fake, None, fake, fake, ctypes.byref(ts), fake, None,
                              fake, 1 << 40, None)
    assert st == M.MINF_EINVAL
    st = lib.minf_sparse_attn(ctypes.byref(p), h, fake, fake, fake, fake, fake, ctypes.byref(ts), fake, None,
                              fake, 1 << 40, None)
    assert st == M.MINF_EINVAL          # VS head without tile lists
    assert "tile" in lib.minf_last_error().decode()
    # exact slash pairs need the two bitmaps
    p1 = _prob(slash_tile=1)
    ts = M.MinfTiles(*([fake] * 10 + [None, None] + [fake] * 3))
    st = lib.minf_build_tiles(ctypes.byref(p1), h, fake, fake, fake, fake, ctypes.byref(ts), fake, 1 << 40, None)
    assert st == M.MINF_EINVAL and "slash_bits" in lib.minf_last_error().decode()
    st = lib.minf_sparse_attn(ctypes.byref(p1), h, fake, fake, fake, fake, fake, ctypes.byref(ts), fake, None,
                              fake, 1 << 40, None)
    assert st == M.MINF_EINVAL and "slash_bits" in lib.minf_last_error().decode()
    # a Vertical-Slash head needs the tail list and the packed-chunk counts
    ts = M.MinfTiles(*([fake] * 12 + [None, fake, fake]))
    st = lib.minf_build_tiles(ctypes.byref(p), h, fake, fake, fake, fake, ctypes.byref(ts), fake, 1 << 40, None)
    assert st == M.MINF_EINVAL and "tail" in lib.minf_last_error().decode()
    st = lib.minf_sparse_attn(ctypes.byref(p), h, fake, fake, fake, fake, fake, ctypes.byref(ts), fake, None,
                              fake, 1 << 40, None)
    assert st == M.MINF_EINVAL


def test_static_attention_refuses_oversized_problems(lib):
    """minf_sparse_attn_static keeps its scheduler scratch in a fixed 8 MiB
    device array: a problem needing more is refused before any GPU call (the
    fake pointers are never dereferenced)."""
    p = _prob(B=64, Hq=64, Hkv=8, n=1 << 20)
    h = M.make_heads([gen.ashape(16, 100)] * 64)
    fake = 0x1000
    ts = M.MinfTiles()
    st = lib.minf_sparse_attn_static(ctypes.byref(p), h, fake, fake, fake, None, None, ctypes.byref(ts), fake, None,
                                     None)
    assert st == M.MINF_EWORKSPACE
    assert "scratch" in lib.minf_last_error().decode()
    st = lib.minf_sparse_attn_static(ctypes.byref(_prob()), M.make_heads(HEADS), None, fake, fake, fake, fake,
                                     ctypes.byref(ts), fake, None, None)
    assert st == M.MINF_EINVAL


def test_no_work_for_absent_kinds(lib):
    """A layer without VS heads makes minf_vs_index a no-op that succeeds
    (and the same for BS); nothing is queued, so no GPU is needed."""
    p = _prob()
    h = M.make_heads([gen.ashape(4, 8)] * 4)
    assert lib.minf_vs_index(ctypes.byref(p), h, None, None, None, None, None, None, None, 0, None) == M.MINF_OK
    assert lib.minf_bs_index(ctypes.byref(p), h, None, None, None, None, None, 0, None) == M.MINF_OK


def test_timing_rejects_bad_arguments(lib):
    # argument checks answer before any event is created
    assert lib.minf_timing_start(0) == M.MINF_EINVAL
    assert lib.minf_timing_start(65537) == M.MINF_EINVAL
    cnt = ctypes.c_int32(-1)
    assert lib.minf_timing_read(None, 0, ctypes.byref(cnt)) == M.MINF_EINVAL   # no timing started
    assert lib.minf_timing_read(None, 4, ctypes.byref(cnt)) == M.MINF_EINVAL   # null output array
    assert lib.minf_timing_read(None, 0, None) == M.MINF_EINVAL


def test_output_error_rejects_bad_arguments(lib):
    """minf_output_error validates before any launch (the fake pointers are
    never dereferenced)."""
    fake = 0x1000
    p = _prob()
    assert lib.minf_output_error(None, fake, fake, fake, None) == M.MINF_EINVAL
    assert lib.minf_output_error(ctypes.byref(p), None, fake, fake, None) == M.MINF_EINVAL
    assert lib.minf_output_error(ctypes.byref(p), fake, None, fake, None) == M.MINF_EINVAL
    assert lib.minf_output_error(ctypes.byref(p), fake, fake, None, None) == M.MINF_EINVAL
    p96 = _prob(dh=96)
    assert lib.minf_output_error(ctypes.byref(p96), fake, fake, fake, None) == M.MINF_EUNSUPPORTED
    p0 = _prob(n=0)
    assert lib.minf_output_error(ctypes.byref(p0), fake, fake, fake, None) == M.MINF_EINVAL
    assert lib.minf_last_error().decode()


def test_ragged_rejects_bad_arguments(lib):
    """minf_prefill_ragged validates lengths, pointers and the workspace
    before any launch (the fake pointers are never dereferenced)."""
    fake = 0x1000
    p = _prob(B=3)
    h = M.make_heads(HEADS)
    need = M.minf_ragged_ws_bytes(p, h, [10, 1000, 7])
    one = M.minf_query_sizes(_prob(B=1), h)
    assert need >= one.ws_bytes
    # the workspace grows with the lengths (every sample keeps its own lists)
    assert M.minf_ragged_ws_bytes(p, h, [10, 20, 7]) < need
    out = ctypes.c_int64(0)
    assert lib.minf_ragged_ws_bytes(ctypes.byref(p), h, None, ctypes.byref(out)) == M.MINF_EINVAL
    assert lib.minf_ragged_ws_bytes(ctypes.byref(p), h, (ctypes.c_int32 * 3)(10, 1001, 7),
                                    ctypes.byref(out)) == M.MINF_EINVAL
    def call(lens, Q=fake, O=fake, status=fake, ws=fake, ws_bytes=need):
        arr = None if lens is None else (ctypes.c_int32 * len(lens))(*lens)
        return lib.minf_prefill_ragged(ctypes.byref(p), h, arr, Q, fake, fake, O, None, None, status, ws, ws_bytes,
                                       None)
    assert call(None) == M.MINF_EINVAL
    assert call([10, 0, 7]) == M.MINF_EINVAL              # an empty sequence
    assert call([10, 1001, 7]) == M.MINF_EINVAL           # longer than n
    assert "length" in lib.minf_last_error().decode()
    assert call([10, 1000, 7], Q=None) == M.MINF_EINVAL
    assert call([10, 1000, 7], O=None) == M.MINF_EINVAL
    assert call([10, 1000, 7], status=None) == M.MINF_EINVAL
    assert call([10, 1000, 7], ws=None) == M.MINF_EWORKSPACE
    assert call([10, 1000, 7], ws_bytes=need - 1) == M.MINF_EWORKSPACE
    # a bad head table is refused like everywhere else
    bad = M.make_heads([gen.HeadCfg(7)] + HEADS[1:])
    assert lib.minf_prefill_ragged(ctypes.byref(p), bad, (ctypes.c_int32 * 3)(1, 2, 3), fake, fake, fake, fake,
                                   None, None, fake, fake, need, None) == M.MINF_EINVAL
