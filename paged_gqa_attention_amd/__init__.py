"""Python binding of libpaged_attn.so (gfx950 paged grouped-query attention).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  The
functions carry the C ABI's names (``attn_paged_decode``, ``attn_prefill``,
``attn_prefill_blocksparse`` ...) and raise ``AttnError`` with the library's
message on any non-OK status.  There is no fallback: if the shared library
is missing or no gfx950 device is present, the calls fail.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

from . import accounting  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

ATTN_OK, ATTN_ERR_INVALID_ARGUMENT, ATTN_ERR_UNSUPPORTED = 0, 1, 2
ATTN_ERR_WORKSPACE_TOO_SMALL, ATTN_ERR_DEVICE = 3, 4
ATTN_F32, ATTN_F16, ATTN_BF16, ATTN_FP8_E4M3, ATTN_BF8_E5M2 = 0, 1, 2, 3, 4

_DT = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16,
       torch.float8_e4m3fn: ATTN_FP8_E4M3, torch.float8_e5m2: ATTN_BF8_E5M2}

ABI_VERSION = 5   # include/paged_attn.h ATTN_ABI_VERSION
NOALLOC_SCRATCH_BYTES = 16 << 20   # ATTN_NOALLOC_SCRATCH_BYTES

EXPORTED = [
    "attn_abi_version", "attn_open", "attn_open_host_only", "attn_close", "attn_free",
    "attn_paged_decode_plan", "attn_paged_decode_workspace_bytes", "attn_paged_decode",
    "attn_paged_decode_noalloc",
    "attn_prefill", "attn_prefill_blocksparse", "attn_kv_append", "attn_debug_gather_kv",
    "attn_debug_read_probe",
]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class attn_kv(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("k_stride_page", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int32),
        ("pad1", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
        ("k_vscales", ctypes.c_void_p), ("v_vscales", ctypes.c_void_p),
        ("vscale_stride_page", ctypes.c_int64), ("vscale_stride_head", ctypes.c_int64),
        ("k_fragments", ctypes.c_void_p), ("v_fragments", ctypes.c_void_p),
        ("fragment_pages_log2", ctypes.c_int32), ("num_fragments", ctypes.c_int32),
    ]


class attn_io(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("q_rows", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_row", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("o", ctypes.c_void_p), ("o_dtype", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("o_stride_b", ctypes.c_int64), ("o_stride_row", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
    ]


class attn_opts(ctypes.Structure):
    _fields_ = [
        ("softmax_scale", ctypes.c_float), ("num_splits", ctypes.c_int32),
        ("sinks", ctypes.c_void_p), ("block_mask", ctypes.c_void_p),
        ("mask_heads", ctypes.c_int32), ("mask_block", ctypes.c_int32),
        ("mask_q_blocks", ctypes.c_int32), ("mask_k_blocks", ctypes.c_int32),
        ("rows_per_seq", ctypes.c_void_p),
    ]


class attn_kv_rows(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("n_new", ctypes.c_int32), ("pad0", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_row", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the shared library (fails loudly if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise AttnError(ATTN_ERR_DEVICE, f"{path} is not built; run "
                        "`python -m paged_gqa_attention_amd.build`")
    lib = ctypes.CDLL(path)
    lib.attn_abi_version.restype = ctypes.c_int
    if lib.attn_abi_version() != ABI_VERSION:
        raise AttnError(ATTN_ERR_DEVICE, f"{path} has ABI {lib.attn_abi_version()}, the binding "
                        f"expects {ABI_VERSION}: rebuild it")
    P = ctypes.POINTER
    vp, st, cp = ctypes.c_void_p, ctypes.c_int, P(ctypes.c_char_p)
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_open.argtypes = [ctypes.c_int, P(vp), cp]
    lib.attn_open.restype = st
    lib.attn_open_host_only.argtypes = [ctypes.c_int, P(vp), cp]
    lib.attn_open_host_only.restype = st
    lib.attn_close.argtypes = [vp]
    lib.attn_close.restype = None
    lib.attn_free.argtypes = [vp]
    lib.attn_free.restype = None
    lib.attn_paged_decode_plan.argtypes = [vp, P(attn_io), P(attn_kv), P(attn_opts),
                                           P(ctypes.c_int32), P(ctypes.c_int32),
                                           P(ctypes.c_size_t), cp]
    lib.attn_paged_decode_plan.restype = st
    lib.attn_paged_decode_workspace_bytes.argtypes = [vp, P(attn_io), P(attn_kv), P(attn_opts)]
    lib.attn_paged_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_paged_decode.argtypes = [vp, P(attn_io), P(attn_kv), P(attn_opts), vp,
                                      ctypes.c_size_t, vp, cp]
    lib.attn_paged_decode.restype = st
    lib.attn_paged_decode_noalloc.argtypes = [vp, P(attn_io), P(attn_kv), P(attn_opts), vp, cp]
    lib.attn_paged_decode_noalloc.restype = st
    for name in ("attn_prefill", "attn_prefill_blocksparse"):
        f = getattr(lib, name)
        f.argtypes = [vp, P(attn_io), P(attn_kv), P(attn_opts), vp, cp]
        f.restype = st
    lib.attn_debug_gather_kv.argtypes = [vp, P(attn_kv), ctypes.c_int32, ctypes.c_int32, vp, vp,
                                         vp, cp]
    lib.attn_debug_gather_kv.restype = st
    lib.attn_kv_append.argtypes = [vp, P(attn_kv), P(attn_kv_rows), vp, cp]
    lib.attn_kv_append.restype = st
    lib.attn_debug_read_probe.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int32, vp, vp, vp, cp]
    lib.attn_debug_read_probe.restype = st
    _lib = lib
    return lib


def _check(status: int, err: ctypes.c_char_p):
    if status != ATTN_OK:
        msg = err.value.decode() if err.value else "(no message)"
        if err.value:
            _lib.attn_free(ctypes.cast(err, ctypes.c_void_p))
        raise AttnError(status, msg)


def attn_abi_version() -> int:
    return load_library().attn_abi_version()


class Context:
    """An open attn_ctx (closed on garbage collection)."""

    def __init__(self, handle: int):
        self.handle = handle

    def close(self):
        if self.handle:
            load_library().attn_close(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def attn_open(device: int = 0) -> Context:
    lib = load_library()
    h = ctypes.c_void_p()
    err = ctypes.c_char_p()
    _check(lib.attn_open(device, ctypes.byref(h), ctypes.byref(err)), err)
    return Context(h.value)


def attn_open_host_only(num_cus: int = 256) -> Context:
    lib = load_library()
    h = ctypes.c_void_p()
    err = ctypes.c_char_p()
    _check(lib.attn_open_host_only(num_cus, ctypes.byref(h), ctypes.byref(err)), err)
    return Context(h.value)


def attn_close(ctx: Context):
    ctx.close()


# ---- marshalling helpers -----------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, f"unsupported tensor dtype {t.dtype}")
    return _DT[t.dtype]


def make_kv(k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
            seq_lens: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0,
            k_vscales: Optional[torch.Tensor] = None,
            v_vscales: Optional[torch.Tensor] = None,
            k_fragments: Optional[torch.Tensor] = None, v_fragments: Optional[torch.Tensor] = None,
            fragment_pages_log2: int = 0, num_pages: Optional[int] = None) -> attn_kv:
    """K pool [num_pages][Hkv][16][d], V pool [num_pages][Hkv][d][16] (any strides on
    the first two dims, tiles contiguous), page_table int32 [B][stride], seq_lens int32 [B].
    Optional per-vector scale pools (8-bit K/V) k_vscales / v_vscales: float32
    [num_pages][Hkv][16] with the 16 slots contiguous and equal strides.

    Fragmented pools: k_fragments / v_fragments are int64 device tensors of
    fragment addresses (``tensor.data_ptr()`` of each fragment), each fragment
    holding 2^fragment_pages_log2 pages; k_pages / v_pages then describe one
    fragment's layout (dtype and strides) and ``num_pages`` gives the pool size."""
    if k_pages.dim() != 4 or v_pages.dim() != 4:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "K/V pools must be 4-D")
    n, hkv, page, d = k_pages.shape
    kv = attn_kv()
    kv.k_pages, kv.v_pages = _ptr(k_pages), _ptr(v_pages)
    if (k_fragments is None) != (v_fragments is None):
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "k_fragments and v_fragments go together here")
    if k_fragments is not None:
        if k_fragments.dtype != torch.int64 or v_fragments.dtype != torch.int64 or \
           k_fragments.shape != v_fragments.shape or k_fragments.dim() != 1:
            raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "fragment tables must be int64 [num_fragments]")
        if num_pages is None or n != 1 << fragment_pages_log2:
            raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "fragmented pools: k_pages describes one "
                            "fragment of 2^fragment_pages_log2 pages; give num_pages")
        kv.k_pages = kv.v_pages = None
        kv.k_fragments, kv.v_fragments = _ptr(k_fragments), _ptr(v_fragments)
        kv.fragment_pages_log2 = int(fragment_pages_log2)
        kv.num_fragments = k_fragments.shape[0]
        n = int(num_pages)
    else:
        kv.k_fragments = kv.v_fragments = None
        kv.fragment_pages_log2 = kv.num_fragments = 0
    kv.dtype = _dtype(k_pages)
    kv.num_pages, kv.page_size, kv.num_kv_heads, kv.head_dim = n, page, hkv, d
    kv.k_stride_page, kv.k_stride_head = k_pages.stride(0), k_pages.stride(1)
    kv.v_stride_page, kv.v_stride_head = v_pages.stride(0), v_pages.stride(1)
    if (k_pages.stride(2), k_pages.stride(3)) != (d, 1) or \
       (v_pages.stride(2), v_pages.stride(3)) != (page, 1) or \
       tuple(v_pages.shape) != (k_pages.shape[0], hkv, d, page) or v_pages.dtype != k_pages.dtype:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "K/V page tiles must be contiguous "
                        "[16][d] (K) and [d][16] (V) of one dtype")
    kv.k_scale, kv.v_scale = float(k_scale), float(v_scale)
    if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "page_table and seq_lens must be int32")
    if page_table.stride(1) != 1:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "page_table rows must be contiguous")
    kv.page_table = _ptr(page_table)
    kv.page_table_stride = page_table.stride(0)
    kv.seq_lens = _ptr(seq_lens)
    if (k_vscales is None) != (v_vscales is None):
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "k_vscales and v_vscales go together")
    if k_vscales is not None:
        for t in (k_vscales, v_vscales):
            if t.dtype != torch.float32 or t.dim() != 3 or t.shape[0] != n or \
               t.shape[1] != hkv or t.shape[2] != page or t.stride(2) != 1:
                raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "per-vector scales must be float32 "
                                "[num_pages][Hkv][16] with contiguous slots")
        if k_vscales.stride() != v_vscales.stride():
            raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "k_vscales and v_vscales need equal strides")
        kv.k_vscales, kv.v_vscales = _ptr(k_vscales), _ptr(v_vscales)
        kv.vscale_stride_page, kv.vscale_stride_head = k_vscales.stride(0), k_vscales.stride(1)
    else:
        kv.k_vscales = kv.v_vscales = None
        kv.vscale_stride_page = kv.vscale_stride_head = 0
    kv._keep = (k_pages, v_pages, page_table, seq_lens, k_vscales, v_vscales, k_fragments,
                v_fragments)
    return kv


def make_rows(k: torch.Tensor, v: torch.Tensor) -> attn_kv_rows:
    """New K/V rows [B][n_new][Hkv][d] (head_dim contiguous, k and v of one layout)."""
    if k.dim() != 4 or v.shape != k.shape or v.dtype != k.dtype or v.stride() != k.stride():
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "k and v must be [B][n_new][Hkv][d] of one layout")
    if k.stride(3) != 1:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "head_dim must be contiguous")
    r = attn_kv_rows()
    r.k, r.v, r.dtype = _ptr(k), _ptr(v), _dtype(k)
    r.batch, r.n_new = k.shape[0], k.shape[1]
    r.stride_b, r.stride_row, r.stride_head = k.stride(0), k.stride(1), k.stride(2)
    r._keep = (k, v)     # the descriptor holds raw pointers: keep the tensors alive with it
    return r


def make_io(q: torch.Tensor, o: torch.Tensor, lse: Optional[torch.Tensor] = None) -> attn_io:
    """Q and O as [B][rows][Hq][d] (head_dim contiguous); lse float32 [B][Hq][rows]."""
    if q.dim() != 4 or o.shape != q.shape:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "q and o must be [B][rows][Hq][d] of one shape")
    if q.stride(3) != 1 or o.stride(3) != 1:
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "head_dim must be contiguous")
    io = attn_io()
    io.q, io.q_dtype = _ptr(q), _dtype(q)
    io.batch, io.q_rows, io.num_q_heads = q.shape[0], q.shape[1], q.shape[2]
    io.q_stride_b, io.q_stride_row, io.q_stride_head = q.stride(0), q.stride(1), q.stride(2)
    io.o, io.o_dtype = _ptr(o), _dtype(o)
    io.o_stride_b, io.o_stride_row, io.o_stride_head = o.stride(0), o.stride(1), o.stride(2)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or \
           tuple(lse.shape) != (q.shape[0], q.shape[2], q.shape[1]):
            raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "lse must be float32 [B][Hq][rows]")
    io.lse = _ptr(lse)
    io._keep = (q, o, lse)
    return io


def make_opts(softmax_scale: float = 0.0, sinks: Optional[torch.Tensor] = None,
              block_mask: Optional[torch.Tensor] = None, mask_block: int = 128,
              num_splits: int = 0, rows_per_seq: Optional[torch.Tensor] = None) -> attn_opts:
    """rows_per_seq: optional int32 [B], the query rows of each sequence (ragged)."""
    op = attn_opts()
    if rows_per_seq is not None and (rows_per_seq.dtype != torch.int32 or
                                     not rows_per_seq.is_contiguous()):
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "rows_per_seq must be contiguous int32 [B]")
    op.rows_per_seq = _ptr(rows_per_seq)
    op.softmax_scale = float(softmax_scale)
    op.num_splits = int(num_splits)
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "sinks must be contiguous float32 [Hq]")
    op.sinks = _ptr(sinks)
    if block_mask is not None:
        if block_mask.dtype != torch.uint8 or block_mask.dim() != 4 or not block_mask.is_contiguous():
            raise AttnError(ATTN_ERR_INVALID_ARGUMENT, "block_mask must be contiguous uint8 "
                            "[B][mask_heads][q_blocks][k_blocks]")
        op.block_mask = _ptr(block_mask)
        op.mask_heads, op.mask_q_blocks, op.mask_k_blocks = (block_mask.shape[1],
                                                             block_mask.shape[2],
                                                             block_mask.shape[3])
    else:
        op.block_mask = None
        op.mask_heads, op.mask_q_blocks, op.mask_k_blocks = 1, 1, 1
    op.mask_block = int(mask_block)
    op._keep = (sinks, block_mask, rows_per_seq)
    return op


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream, device) -> torch.cuda.Stream:
    """The stream a convenience call enqueues on, as a torch stream object (a raw
    handle is wrapped), so that its temporaries are allocated on that stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


# ---- the C ABI calls ----------------------------------------------------------------

def attn_paged_decode_plan(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts):
    """(num_splits, tokens_per_split, workspace_bytes) the library will use."""
    lib = load_library()
    P, T, W = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    err = ctypes.c_char_p()
    _check(lib.attn_paged_decode_plan(ctx.handle, ctypes.byref(io), ctypes.byref(kv),
                                      ctypes.byref(opts), ctypes.byref(P), ctypes.byref(T),
                                      ctypes.byref(W), ctypes.byref(err)), err)
    return P.value, T.value, W.value


def attn_paged_decode_workspace_bytes(ctx: Context, io: attn_io, kv: attn_kv,
                                      opts: attn_opts) -> int:
    return load_library().attn_paged_decode_workspace_bytes(ctx.handle, ctypes.byref(io),
                                                            ctypes.byref(kv), ctypes.byref(opts))


def attn_paged_decode(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts,
                      workspace: torch.Tensor, stream=None):
    lib = load_library()
    err = ctypes.c_char_p()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_paged_decode(ctx.handle, ctypes.byref(io), ctypes.byref(kv),
                                 ctypes.byref(opts), workspace.data_ptr(), nbytes,
                                 _stream_ptr(stream), ctypes.byref(err)), err)


def attn_paged_decode_noalloc(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts,
                              stream=None):
    """attn_paged_decode with the library's device-resident scratch (no workspace,
    no allocation); calls that overlap on one device race."""
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_paged_decode_noalloc(ctx.handle, ctypes.byref(io), ctypes.byref(kv),
                                         ctypes.byref(opts), _stream_ptr(stream),
                                         ctypes.byref(err)), err)


def attn_prefill(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts, stream=None):
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_prefill(ctx.handle, ctypes.byref(io), ctypes.byref(kv), ctypes.byref(opts),
                            _stream_ptr(stream), ctypes.byref(err)), err)


def attn_prefill_blocksparse(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts,
                             stream=None):
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_prefill_blocksparse(ctx.handle, ctypes.byref(io), ctypes.byref(kv),
                                        ctypes.byref(opts), _stream_ptr(stream),
                                        ctypes.byref(err)), err)


def attn_kv_append(ctx: Context, kv: attn_kv, rows: attn_kv_rows, stream=None):
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_kv_append(ctx.handle, ctypes.byref(kv), ctypes.byref(rows), _stream_ptr(stream),
                              ctypes.byref(err)), err)


def attn_debug_gather_kv(ctx: Context, kv: attn_kv, b: int, seq_len: int, k_out: torch.Tensor,
                         v_out: torch.Tensor, stream=None):
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_debug_gather_kv(ctx.handle, ctypes.byref(kv), b, seq_len, _ptr(k_out),
                                    _ptr(v_out), _stream_ptr(stream), ctypes.byref(err)), err)


def attn_debug_read_probe(ctx: Context, buf: torch.Tensor, pattern: int,
                          tile_order: Optional[torch.Tensor], sink: torch.Tensor, stream=None):
    """Read-only HBM probe over ``buf`` (pattern 0 contiguous, 1 4 KiB tiles and
    2 2 KiB tiles in ``tile_order``); a measurement hook."""
    lib = load_library()
    err = ctypes.c_char_p()
    _check(lib.attn_debug_read_probe(ctx.handle, _ptr(buf), buf.numel() * buf.element_size(),
                                     pattern, _ptr(tile_order), _ptr(sink), _stream_ptr(stream),
                                     ctypes.byref(err)), err)


# ---- convenience: whole calls on torch tensors -----------------------------------------

def decode_workspace(ctx: Context, io: attn_io, kv: attn_kv, opts: attn_opts, device):
    """A decode workspace of the size the library asks for."""
    nb = attn_paged_decode_workspace_bytes(ctx, io, kv, opts)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def paged_decode(ctx: Context, q, k_pages, v_pages, page_table, seq_lens, *, k_scale=1.0,
                 v_scale=1.0, softmax_scale=0.0, sinks=None, out=None, out_dtype=None,
                 lse=None, num_splits=0, workspace=None, stream=None, rows_per_seq=None,
                 k_vscales=None, v_vscales=None):
    """Decode / verify rows ``q`` [B][R][Hq][d]; returns the output tensor.  With
    ``rows_per_seq`` (int32 [B]) sequence b has only its first rows_per_seq[b] rows;
    ``k_vscales``/``v_vscales`` are per-vector scale pools of an 8-bit cache.

    The call is enqueued on ``stream`` (default: the current stream).  The output
    and a workspace this function allocates are allocated on that stream, so the
    caching allocator does not hand the workspace to other work before the call's
    kernels have finished with it."""
    s = _torch_stream(stream, q.device)
    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty(q.shape, dtype=out_dtype or q.dtype,
                                                     device=q.device)
        io = make_io(q, o, lse)
        kv = make_kv(k_pages, v_pages, page_table, seq_lens, k_scale, v_scale, k_vscales,
                     v_vscales)
        op = make_opts(softmax_scale, sinks, None, 128, num_splits, rows_per_seq)
        if workspace is None:
            workspace = decode_workspace(ctx, io, kv, op, q.device)
        attn_paged_decode(ctx, io, kv, op, workspace, s)
    return o


def prefill(ctx: Context, q, k_pages, v_pages, page_table, seq_lens, *, k_scale=1.0,
            v_scale=1.0, softmax_scale=0.0, sinks=None, out=None, out_dtype=None, lse=None,
            block_mask=None, mask_block=128, stream=None, rows_per_seq=None, k_vscales=None,
            v_vscales=None):
    """Causal (optionally block-sparse) prefill of ``q`` [B][S_q][Hq][d]; with
    ``rows_per_seq`` (int32 [B]) sequence b has only its first rows_per_seq[b] rows;
    ``k_vscales``/``v_vscales`` are per-vector scale pools of an 8-bit cache.  The
    call is enqueued on ``stream`` (default: the current stream), where the output
    is allocated too."""
    s = _torch_stream(stream, q.device)
    with torch.cuda.stream(s):
        o = out if out is not None else torch.empty(q.shape, dtype=out_dtype or q.dtype,
                                                     device=q.device)
        io = make_io(q, o, lse)
        kv = make_kv(k_pages, v_pages, page_table, seq_lens, k_scale, v_scale, k_vscales,
                     v_vscales)
        op = make_opts(softmax_scale, sinks, block_mask, mask_block, rows_per_seq=rows_per_seq)
        if block_mask is None:
            attn_prefill(ctx, io, kv, op, s)
        else:
            attn_prefill_blocksparse(ctx, io, kv, op, s)
    return o
