"""Python binding of libminf (MInference-style dynamic-sparse prefill on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libminf.so (built in-tree by ``long_context_prefill_amd.build``).  PyTorch is
used for device memory and streams; tensors are passed as raw device
pointers.  If the shared library is missing, importing the entry points
raises - there is no fallback implementation.

Entry points (same names and argument order as include/minf.h):
    minf_query_sizes(prob, heads) -> MinfSizes
    minf_vs_index(prob, heads, Q, K, vert_idx, slash_idx, vert_score, slash_score, ws, stream=None)
    minf_vs_index_fused(...)   same, the proxy in one launch
    minf_bs_index(prob, heads, Q, K, blk_idx, blk_cnt, ws, stream=None)
    minf_build_tiles(prob, heads, vert_idx, slash_idx, blk_idx, blk_cnt, tiles, ws, stream=None)
    minf_sparse_attn(prob, heads, Q, K, V, blk_idx, blk_cnt, tiles, O, lse, ws, stream=None)
    minf_sparse_attn_static(...)  the same without a workspace (static scratch)
    minf_output_error(prob, O, O_ref, err, stream=None)
    minf_captured_mass(prob, lse, lse_ref, mass, stream=None)
    minf_ragged_ws_bytes(prob, heads, seq_lens) -> int
    minf_prefill_ragged(prob, heads, seq_lens, Q, K, V, O, lse, kept_edges, status, ws, stream=None)
The offline pattern search that drives them on calibration input is in
long_context_prefill_amd.search.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libminf.so")

MINF_OK, MINF_EINVAL, MINF_EUNSUPPORTED, MINF_EWORKSPACE, MINF_ECAPACITY, MINF_EHIP = range(6)
MINF_F32, MINF_BF16 = 0, 1
MINF_ASHAPE, MINF_VSLASH, MINF_BSPARSE = 0, 1, 2
MINF_FORCE_FIRST_BLOCK, MINF_FORCE_DIAG_BLOCK = 1, 2
MINF_DEV_BAD_VERTICAL, MINF_DEV_BAD_SLASH, MINF_DEV_BAD_BLOCK, MINF_DEV_CAPACITY = 1, 2, 4, 8
MINF_DEV_WAIT_EXHAUSTED = 16
MINF_TAIL_PAD = 1 << 30

EXPORTED = ["minf_query_sizes", "minf_vs_index", "minf_vs_index_fused", "minf_bs_index", "minf_build_tiles",
            "minf_sparse_attn", "minf_sparse_attn_static", "minf_output_error", "minf_captured_mass", "minf_ragged_ws_bytes",
            "minf_prefill_ragged", "minf_timing_start",
            "minf_timing_read", "minf_status_string", "minf_last_error", "minf_version"]


class MinfError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"minf status {status}: {msg}")
        self.status = status


class MinfProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("n", ctypes.c_int32), ("dh", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("block", ctypes.c_int32),
                ("slash_tile", ctypes.c_int32)]


class MinfHeadCfg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("last_q", ctypes.c_int32), ("n_vertical", ctypes.c_int32), ("n_slash", ctypes.c_int32),
                ("topk_blocks", ctypes.c_int32), ("force_flags", ctypes.c_int32)]


class MinfSizes(ctypes.Structure):
    _fields_ = [("nq", ctypes.c_int64), ("max_v", ctypes.c_int64), ("max_s", ctypes.c_int64),
                ("max_kb", ctypes.c_int64), ("max_chunks", ctypes.c_int64), ("ws_bytes", ctypes.c_int64),
                ("bits_words", ctypes.c_int64), ("max_tail", ctypes.c_int64)]


class MinfTiles(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("span_lo", "span_hi", "span_cnt", "chunk_lo", "chunk_hi", "chunk_cnt",
                 "cols", "col_cnt", "kept_edges", "status", "slash_bits", "col_bits", "tail_x", "tail_cnt",
                 "pk_cnt")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libminf.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libminf.so not found at {path}; build it with "
                          f"`python -m long_context_prefill_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.minf_query_sizes.argtypes = [P(MinfProblem), P(MinfHeadCfg), P(MinfSizes)]
    lib.minf_vs_index.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.minf_vs_index_fused.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        vp, vp]
    lib.minf_bs_index.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.minf_build_tiles.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, P(MinfTiles), vp,
                                     ctypes.c_size_t, vp]
    lib.minf_sparse_attn.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, vp, P(MinfTiles), vp, vp,
                                     vp, ctypes.c_size_t, vp]
    lib.minf_sparse_attn_static.argtypes = [P(MinfProblem), P(MinfHeadCfg), vp, vp, vp, vp, vp, P(MinfTiles), vp,
                                            vp, vp]
    lib.minf_output_error.argtypes = [P(MinfProblem), vp, vp, vp, vp]
    lib.minf_captured_mass.argtypes = [P(MinfProblem), vp, vp, vp, vp]
    lib.minf_ragged_ws_bytes.argtypes = [P(MinfProblem), P(MinfHeadCfg), P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.minf_prefill_ragged.argtypes = [P(MinfProblem), P(MinfHeadCfg), P(ctypes.c_int32), vp, vp, vp, vp, vp, vp, vp,
                                        vp, ctypes.c_size_t, vp]
    for f in ("minf_query_sizes", "minf_vs_index", "minf_vs_index_fused", "minf_bs_index", "minf_build_tiles",
              "minf_sparse_attn", "minf_sparse_attn_static",
              "minf_output_error", "minf_captured_mass", "minf_ragged_ws_bytes", "minf_prefill_ragged"):
        getattr(lib, f).restype = ctypes.c_int
    lib.minf_timing_start.argtypes = [ctypes.c_int32]
    lib.minf_timing_start.restype = ctypes.c_int
    lib.minf_timing_read.argtypes = [P(ctypes.c_float), ctypes.c_int32, P(ctypes.c_int32)]
    lib.minf_timing_read.restype = ctypes.c_int
    lib.minf_status_string.argtypes = [ctypes.c_int]
    lib.minf_status_string.restype = ctypes.c_char_p
    lib.minf_last_error.argtypes = []
    lib.minf_last_error.restype = ctypes.c_char_p
    lib.minf_version.argtypes = []
    lib.minf_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling

def make_problem(B, Hq, Hkv, n, dh, in_dtype="bf16", out_dtype="f32", scale=0.0, block=64,
                 slash_tile=64) -> MinfProblem:
    dt = {"f32": MINF_F32, "bf16": MINF_BF16}
    return MinfProblem(B, Hq, Hkv, n, dh, dt[in_dtype], dt[out_dtype], float(scale), block, slash_tile)


def make_heads(heads: Sequence) -> ctypes.Array:
    """Heads as objects with .as_tuple() or as 8-tuples in minf_head_cfg order."""
    arr = (MinfHeadCfg * max(1, len(heads)))()
    for i, h in enumerate(heads):
        t = h.as_tuple() if hasattr(h, "as_tuple") else tuple(h)
        arr[i] = MinfHeadCfg(*[int(x) for x in t])
    return arr


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL); only contiguous tensors."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("minf takes contiguous tensors only")
    return t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status):
    if status != MINF_OK:
        lib = load_library()
        raise MinfError(status, lib.minf_last_error().decode())


def tiles_struct(tiles: dict) -> MinfTiles:
    return MinfTiles(*[_ptr(tiles.get(f)) for f, _ in MinfTiles._fields_])


# ---------------------------------------------------------------- entry points

def minf_query_sizes(prob: MinfProblem, heads) -> MinfSizes:
    lib = load_library()
    out = MinfSizes()
    _check(lib.minf_query_sizes(ctypes.byref(prob), heads, ctypes.byref(out)))
    return out


def minf_vs_index(prob, heads, Q, K, vert_idx, slash_idx, vert_score=None, slash_score=None, ws=None,
                  stream=None):
    lib = load_library()
    _check(lib.minf_vs_index(ctypes.byref(prob), heads, _ptr(Q), _ptr(K), _ptr(vert_idx), _ptr(slash_idx),
                             _ptr(vert_score), _ptr(slash_score), _ptr(ws), _nbytes(ws), _stream(stream)))


def minf_vs_index_fused(prob, heads, Q, K, vert_idx, slash_idx, vert_score=None, slash_score=None, ws=None,
                        status=None, stream=None):
    lib = load_library()
    _check(lib.minf_vs_index_fused(ctypes.byref(prob), heads, _ptr(Q), _ptr(K), _ptr(vert_idx), _ptr(slash_idx),
                                   _ptr(vert_score), _ptr(slash_score), _ptr(ws), _nbytes(ws), _ptr(status),
                                   _stream(stream)))


def minf_bs_index(prob, heads, Q, K, blk_idx, blk_cnt, ws=None, stream=None):
    lib = load_library()
    _check(lib.minf_bs_index(ctypes.byref(prob), heads, _ptr(Q), _ptr(K), _ptr(blk_idx), _ptr(blk_cnt),
                             _ptr(ws), _nbytes(ws), _stream(stream)))


def minf_build_tiles(prob, heads, vert_idx, slash_idx, blk_idx, blk_cnt, tiles: dict, ws=None, stream=None):
    lib = load_library()
    ts = tiles_struct(tiles)
    _check(lib.minf_build_tiles(ctypes.byref(prob), heads, _ptr(vert_idx), _ptr(slash_idx), _ptr(blk_idx),
                                _ptr(blk_cnt), ctypes.byref(ts), _ptr(ws), _nbytes(ws), _stream(stream)))


def minf_sparse_attn(prob, heads, Q, K, V, blk_idx, blk_cnt, tiles: Optional[dict], O, lse=None, ws=None,
                     stream=None):
    lib = load_library()
    ts = tiles_struct(tiles or {})
    _check(lib.minf_sparse_attn(ctypes.byref(prob), heads, _ptr(Q), _ptr(K), _ptr(V), _ptr(blk_idx),
                                _ptr(blk_cnt), ctypes.byref(ts), _ptr(O), _ptr(lse), _ptr(ws), _nbytes(ws),
                                _stream(stream)))


def minf_sparse_attn_static(prob, heads, Q, K, V, blk_idx, blk_cnt, tiles: Optional[dict], O, lse=None,
                            stream=None):
    lib = load_library()
    ts = tiles_struct(tiles or {})
    _check(lib.minf_sparse_attn_static(ctypes.byref(prob), heads, _ptr(Q), _ptr(K), _ptr(V), _ptr(blk_idx),
                                       _ptr(blk_cnt), ctypes.byref(ts), _ptr(O), _ptr(lse), _stream(stream)))


def minf_output_error(prob, O, O_ref, err, stream=None):
    """err (device, 2 * B * Hq float64) <- per head: sum of (O - O_ref)^2 and
    sum of O_ref^2."""
    lib = load_library()
    _check(lib.minf_output_error(ctypes.byref(prob), _ptr(O), _ptr(O_ref), _ptr(err), _stream(stream)))


def minf_captured_mass(prob, lse, lse_ref, mass, stream=None):
    """mass (device, B * Hq float64) <- per head: sum over rows of
    exp(lse - lse_ref)."""
    lib = load_library()
    _check(lib.minf_captured_mass(ctypes.byref(prob), _ptr(lse), _ptr(lse_ref), _ptr(mass), _stream(stream)))


def _lens(seq_lens):
    return (ctypes.c_int32 * max(1, len(seq_lens)))(*[int(x) for x in seq_lens])


def minf_ragged_ws_bytes(prob, heads, seq_lens) -> int:
    """seq_lens: a host sequence of prob.B lengths."""
    lib = load_library()
    out = ctypes.c_int64(0)
    _check(lib.minf_ragged_ws_bytes(ctypes.byref(prob), heads, _lens(seq_lens), ctypes.byref(out)))
    return int(out.value)


def minf_prefill_ragged(prob, heads, seq_lens, Q, K, V, O, lse, kept_edges, status, ws, stream=None):
    """seq_lens: a host sequence of prob.B lengths; tensors packed as
    include/minf.h describes."""
    lib = load_library()
    _check(lib.minf_prefill_ragged(ctypes.byref(prob), heads, _lens(seq_lens), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                                   _ptr(kept_edges), _ptr(status), _ptr(ws), _nbytes(ws), _stream(stream)))


def minf_timing_start(max_calls: int):
    lib = load_library()
    _check(lib.minf_timing_start(int(max_calls)))


def minf_timing_read(cap: int) -> list:
    """Durations (ms) of the main attention kernel of the sparse-attention
    calls made since minf_timing_start, in call order."""
    lib = load_library()
    arr = (ctypes.c_float * max(1, cap))()
    cnt = ctypes.c_int32(0)
    _check(lib.minf_timing_read(arr, int(cap), ctypes.byref(cnt)))
    return [float(arr[i]) for i in range(min(cap, cnt.value))]


# ---------------------------------------------------------------- buffers

def alloc_buffers(prob: MinfProblem, heads, device="cuda"):
    """Allocate (with torch) every index, tile and workspace buffer the four
    calls need, sized by minf_query_sizes.  Returns a dict of tensors."""
    import torch
    sz = minf_query_sizes(prob, heads)
    B, Hq, nq = prob.B, prob.Hq, int(sz.nq)
    i32 = dict(dtype=torch.int32, device=device)
    buf = {
        "sizes": sz,
        "vert_idx": torch.full((B, Hq, int(sz.max_v) or 1), -1, **i32),
        "slash_idx": torch.full((B, Hq, int(sz.max_s)), -1, **i32),
        "blk_idx": torch.full((B, Hq, nq, int(sz.max_kb)), -1, **i32),
        "blk_cnt": torch.zeros((B, Hq, nq), **i32),
        "ws": torch.empty(int(sz.ws_bytes), dtype=torch.uint8, device=device),
        "tiles": {
            "span_lo": torch.zeros((B, Hq, int(sz.max_s)), **i32),
            "span_hi": torch.zeros((B, Hq, int(sz.max_s)), **i32),
            "span_cnt": torch.zeros((B, Hq), **i32),
            "chunk_lo": torch.zeros((B, Hq, int(sz.max_chunks)), **i32),
            "chunk_hi": torch.zeros((B, Hq, int(sz.max_chunks)), **i32),
            "chunk_cnt": torch.zeros((B, Hq, nq), **i32),
            "cols": torch.zeros((B, Hq, nq, int(sz.max_v) or 1), **i32),
            "col_cnt": torch.zeros((B, Hq, nq), **i32),
            "tail_x": torch.zeros((B, Hq, int(sz.max_tail)), **i32),
            "tail_cnt": torch.zeros((B, Hq), **i32),
            "pk_cnt": torch.zeros((B, Hq, nq), **i32),
            "kept_edges": torch.zeros((B, Hq), dtype=torch.int64, device=device),
            "status": torch.zeros(1, **i32),
        },
    }
    if int(sz.bits_words) > 0:
        buf["tiles"]["slash_bits"] = torch.zeros((B, Hq, int(sz.bits_words)), **i32)
        buf["tiles"]["col_bits"] = torch.zeros((B, Hq, int(sz.bits_words)), **i32)
    return buf


def run_layer(prob, heads, Q, K, V, O, lse=None, buf=None, stream=None, vert_score=None, slash_score=None):
    """The whole hot path on one stream: VS index, BS index, tile build and
    sparse attention.  Returns the buffer dict (indices, tiles, kept edges)."""
    if buf is None:
        buf = alloc_buffers(prob, heads, Q.device)
    t = buf["tiles"]
    minf_vs_index(prob, heads, Q, K, buf["vert_idx"], buf["slash_idx"], vert_score, slash_score, buf["ws"], stream)
    minf_bs_index(prob, heads, Q, K, buf["blk_idx"], buf["blk_cnt"], buf["ws"], stream)
    minf_build_tiles(prob, heads, buf["vert_idx"], buf["slash_idx"], buf["blk_idx"], buf["blk_cnt"], t,
                     buf["ws"], stream)
    minf_sparse_attn(prob, heads, Q, K, V, buf["blk_idx"], buf["blk_cnt"], t, O, lse, buf["ws"], stream)
    return buf
