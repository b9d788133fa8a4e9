"""FP64 CPU oracle for paged grouped-query attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: loaded by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``.  The attention library never imports it.
The arithmetic lives in ``attn_oracle.c`` (plain C, double precision); this
file only marshals arguments.

Every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_append_oracle.py`` except the readings the pages leave open and
that no mathematics can fix (the FP8 per-tensor scale choice, the rule that
picks a per-vector scale, and the units of the sink logit): those are "parity
unpinned" and are applied identically by the oracle and the GPU path.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double semantics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp,
                               _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("kv_dtype", ctypes.c_int32),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_stride_page", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double),
        ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32), ("q", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
        ("sinks", ctypes.c_void_p),
        ("mask", ctypes.c_void_p),
        ("mask_heads", ctypes.c_int32), ("mask_block", ctypes.c_int32),
        ("mask_nqb", ctypes.c_int32), ("mask_nkb", ctypes.c_int32),
        ("rows_per_seq", ctypes.c_void_p),
        ("k_vs", ctypes.c_void_p), ("v_vs", ctypes.c_void_p),
        ("vs_stride_page", ctypes.c_int64), ("vs_stride_head", ctypes.c_int64),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _lib.orc_decode.restype = ctypes.c_double
        _lib.orc_decode.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64]
        _lib.orc_decode_array.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p]
        _lib.orc_gather.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
        _lib.orc_attend_partial.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.orc_merge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                   ctypes.c_void_p]
        _lib.orc_encode_array.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_float, ctypes.c_void_p]
        _lib.orc_vector_scales.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_float, ctypes.c_void_p]
        _lib.orc_encode_vectors.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.orc_attend_rows.restype = ctypes.c_int
        _lib.orc_attend_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int]
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class OracleProblem:
    """Holds CPU-contiguous copies of a ``synth.Problem`` and the C struct."""

    def __init__(self, p):
        cpu = lambda t: None if t is None else t.detach().to("cpu").contiguous()
        self.p = p
        self.k = cpu(p.k_pool)
        self.v = cpu(p.v_pool)
        self.pt = cpu(p.page_table).to(torch.int32)
        self.lens = cpu(p.seq_lens).to(torch.int32)
        self.q = cpu(p.q)
        self.sinks = cpu(p.sinks).to(torch.float32) if p.sinks is not None else None
        self.mask = cpu(p.mask).to(torch.uint8) if p.mask is not None else None
        rps = getattr(p, "rows_per_seq", None)
        self.rows_per_seq = cpu(rps).to(torch.int32) if rps is not None else None
        d, hkv, page = p.head_dim, p.num_kv_heads, self.k.shape[2]
        s = _Problem()
        s.kv_dtype = p.kv_dtype
        s.k_pool = self.k.data_ptr()
        s.v_pool = self.v.data_ptr()
        s.k_stride_page, s.k_stride_head = hkv * page * d, page * d
        s.v_stride_page, s.v_stride_head = hkv * page * d, page * d
        s.num_pages, s.num_kv_heads, s.head_dim, s.page_size = self.k.shape[0], hkv, d, page
        s.k_scale, s.v_scale = float(p.k_scale), float(p.v_scale)
        s.page_table = self.pt.data_ptr()
        s.page_table_stride = self.pt.shape[1]
        s.seq_lens = self.lens.data_ptr()
        s.q_dtype = p.q_dtype
        s.q = self.q.data_ptr()
        s.batch, s.n_q, s.num_q_heads = p.batch, p.q_rows, p.num_q_heads
        s.softmax_scale = float(p.softmax_scale)
        s.sinks = self.sinks.data_ptr() if self.sinks is not None else None
        if self.mask is not None:
            s.mask = self.mask.data_ptr()
            s.mask_heads = self.mask.shape[1]
            s.mask_block = p.mask_block
            s.mask_nqb, s.mask_nkb = self.mask.shape[2], self.mask.shape[3]
        else:
            s.mask = None
            s.mask_heads, s.mask_block, s.mask_nqb, s.mask_nkb = 1, 128, 0, 0
        s.rows_per_seq = self.rows_per_seq.data_ptr() if self.rows_per_seq is not None else None
        kvs, vvs = getattr(p, "k_vs", None), getattr(p, "v_vs", None)
        self.k_vs = cpu(kvs).to(torch.float32) if kvs is not None else None
        self.v_vs = cpu(vvs).to(torch.float32) if vvs is not None else None
        if self.k_vs is not None:
            s.k_vs, s.v_vs = self.k_vs.data_ptr(), self.v_vs.data_ptr()
            s.vs_stride_page, s.vs_stride_head = hkv * page, page
        else:
            s.k_vs = s.v_vs = None
            s.vs_stride_page = s.vs_stride_head = 0
        self.struct = s

    def all_rows(self) -> np.ndarray:
        p = self.p
        b, i, h = np.meshgrid(np.arange(p.batch), np.arange(p.q_rows), np.arange(p.num_q_heads),
                              indexing="ij")
        return np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1).astype(np.int32)


def attend(p, rows: Optional[np.ndarray] = None, threads: Optional[int] = None):
    """Attention rows by definition.

    ``rows`` is an int32 array of (b, i, h) triples (default: every row).
    Returns (o [n][d] float64, lse [n] float64, threads_used)."""
    lib = _load()
    op = p if isinstance(p, OracleProblem) else OracleProblem(p)
    if rows is None:
        rows = op.all_rows()
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
    n = rows.shape[0]
    d = op.p.head_dim
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    used = lib.orc_attend_rows(ctypes.byref(op.struct), n, rows.ctypes.data, o.ctypes.data,
                               lse.ctypes.data, int(threads))
    return o, lse, used


def attend_full(p, threads=None):
    """All rows as arrays shaped like the output: o [B][n_q][Hq][d], lse [B][Hq][n_q]."""
    o, lse, _ = attend(p, None, threads)
    B, R, H, d = p.batch, p.q_rows, p.num_q_heads, p.head_dim
    return o.reshape(B, R, H, d), lse.reshape(B, R, H).transpose(0, 2, 1)


def gather(p, b: int, g: int):
    """Logical (dequantised, scaled) K and V of sequence b, KV head g: [L][d] float64."""
    lib = _load()
    op = p if isinstance(p, OracleProblem) else OracleProblem(p)
    L = min(int(op.lens[b]), op.pt.shape[1] * op.k.shape[2])   # clamped to the capacity
    d = op.p.head_dim
    k = np.zeros((L, d), dtype=np.float64)
    v = np.zeros((L, d), dtype=np.float64)
    lib.orc_gather(ctypes.byref(op.struct), b, g, k.ctypes.data, v.ctypes.data)
    return k, v


def attend_partial(p, b, i, h, j0, j1):
    """Per-partition state (o normalised within the partition, m, l), no sink."""
    lib = _load()
    op = p if isinstance(p, OracleProblem) else OracleProblem(p)
    d = op.p.head_dim
    o = np.zeros((d,), dtype=np.float64)
    m = ctypes.c_double()
    l = ctypes.c_double()
    lib.orc_attend_partial(ctypes.byref(op.struct), b, i, h, j0, j1, o.ctypes.data,
                           ctypes.byref(m), ctypes.byref(l))
    return o, m.value, l.value


def merge(o_parts: np.ndarray, m: Sequence[float], l: Sequence[float], sink=-math.inf):
    """Log-sum-exp merge of partition states plus an optional sink."""
    lib = _load()
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    n, d = o_parts.shape
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.zeros((d,), dtype=np.float64)
    lse = ctypes.c_double()
    lib.orc_merge(n, d, o_parts.ctypes.data, m.ctypes.data, l.ctypes.data, float(sink),
                  o.ctypes.data, ctypes.byref(lse))
    return o, lse.value


def decode_codes(dtype: int, codes: np.ndarray) -> np.ndarray:
    """Decode raw storage codes (uint8/uint16/float32 bit patterns) to float64."""
    lib = _load()
    codes = np.ascontiguousarray(codes)
    out = np.zeros(codes.size, dtype=np.float64)
    lib.orc_decode_array(dtype, codes.ctypes.data, codes.size, out.ctypes.data)
    return out


_CODE_NP = {0: np.uint32, 1: np.uint16, 2: np.uint16, 3: np.uint8, 4: np.uint8}
# largest finite value of the 8-bit formats (e4m3fn, e5m2)
FMAX = {3: 448.0, 4: 57344.0}


def encode(dtype: int, x, scale: float = 1.0) -> np.ndarray:
    """Storage codes of float32 values x / scale in ``dtype`` (F32: the quotient's
    bits): round-to-nearest-even, IEEE overflow to infinity, e4m3fn saturating
    at +-448, e5m2 at +-57344 (attn_oracle.c, "Encoding for the K/V append step")."""
    lib = _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.zeros(x.shape, dtype=_CODE_NP[dtype])
    lib.orc_encode_array(dtype, x.size, x.ctypes.data, float(np.float32(scale)), out.ctypes.data)
    return out


def vector_scales(dtype: int, x) -> np.ndarray:
    """Per-vector scales (float32, one per vector along the last axis of x) of
    an 8-bit format: amax over the finite entries / the format's largest
    finite value, 1 where that is 0."""
    lib = _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    d = x.shape[-1]
    n = x.size // d
    out = np.zeros(x.shape[:-1], dtype=np.float32)
    lib.orc_vector_scales(n, d, x.ctypes.data, float(FMAX[dtype]), out.ctypes.data)
    return out


def encode_vectors(dtype: int, x, scales) -> np.ndarray:
    """Codes of x[..., i] / scales[...] (the scale of each vector along the last axis)."""
    lib = _load()
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    sc = np.ascontiguousarray(np.asarray(scales, dtype=np.float32))
    assert sc.shape == x.shape[:-1]
    d = x.shape[-1]
    out = np.zeros(x.shape, dtype=_CODE_NP[dtype])
    lib.orc_encode_vectors(dtype, x.size // d, d, x.ctypes.data, sc.ctypes.data, out.ctypes.data)
    return out


def kv_append(kv_dtype: int, k_codes: np.ndarray, v_codes: np.ndarray, page_table: np.ndarray,
              seq_lens: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, k_scale: float = 1.0,
              v_scale: float = 1.0, page_size: int = 16, k_vs: Optional[np.ndarray] = None,
              v_vs: Optional[np.ndarray] = None):
    """Expected K/V pools after appending n_new rows per sequence.

    k_codes [pages][Hkv][16][d] and v_codes [pages][Hkv][d][16] hold storage codes;
    k_new / v_new are float32 [B][n_new][Hkv][d] (the source rows, exactly
    widened).  Row i of sequence b lands at position L_b - n_new + i, where
    L_b = seq_lens[b] clamped to the page table's capacity; rows at negative
    positions are dropped.  Everything else in the pools is left as it was.

    With per-vector scale pools k_vs / v_vs (float32 [pages][Hkv][16], 8-bit
    storage, per-tensor scales 1) each new (token, head) vector is encoded
    with its own scale (``vector_scales``), which lands in the scale pool's
    slot; returns (k, v, k_vs, v_vs) then, else (k, v).
    """
    B, n_new = k_new.shape[0], k_new.shape[1]
    cap = page_table.shape[1] * page_size
    per_vector = k_vs is not None
    if per_vector:
        ks_new, vs_new = vector_scales(kv_dtype, k_new), vector_scales(kv_dtype, v_new)
        kc, vc = encode_vectors(kv_dtype, k_new, ks_new), encode_vectors(kv_dtype, v_new, vs_new)
        k_vs, v_vs = k_vs.copy(), v_vs.copy()
    else:
        kc = encode(kv_dtype, k_new, k_scale)
        vc = encode(kv_dtype, v_new, v_scale)
    k_out, v_out = k_codes.copy(), v_codes.copy()
    for b in range(B):
        L = min(int(seq_lens[b]), cap)
        for i in range(n_new):
            pos = L - n_new + i
            if pos < 0:
                continue
            page, slot = int(page_table[b, pos // page_size]), pos % page_size
            k_out[page, :, slot, :] = kc[b, i]
            v_out[page, :, :, slot] = vc[b, i]
            if per_vector:
                k_vs[page, :, slot] = ks_new[b, i]
                v_vs[page, :, slot] = vs_new[b, i]
    return (k_out, v_out, k_vs, v_vs) if per_vector else (k_out, v_out)
