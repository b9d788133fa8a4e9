"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol the header declares, and its argument checking and split planning
behave as documented.  Planning-only contexts never enqueue work."""
import ctypes
import os
import re

import pytest
import torch

import paged_gqa_attention_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status|size_t|int|void)\s+\**(attn_\w+)\s*\(",
                                 src, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(pa.EXPORTED)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.skip("library not built")
    return pa.load_library()


def test_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.attn_abi_version() == 5


def test_open_without_a_gpu_is_a_device_error(lib):
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(pa.AttnError) as e:
        pa.attn_open(0)
    assert e.value.status == pa.ATTN_ERR_DEVICE


class FakeTensor:
    """Shape/stride/pointer stand-in so argument checks can run without device memory."""

    def __init__(self, shape, dtype, ptr=0x10000, strides=None):
        self.shape = tuple(shape)
        self.dtype = dtype
        self._ptr = ptr
        if strides is None:
            strides, acc = [], 1
            for s in reversed(shape):
                strides.append(acc)
                acc *= s
            strides = list(reversed(strides))
        self._strides = tuple(strides)

    def data_ptr(self):
        return self._ptr

    def stride(self, i=None):
        return self._strides if i is None else self._strides[i]

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return True

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()


def _decode_args(B=2, R=1, Hq=8, Hkv=2, d=128, stride=64, dtype=torch.bfloat16, pages=100):
    k = FakeTensor((pages, Hkv, 16, d), dtype, 0x100000)
    v = FakeTensor((pages, Hkv, d, 16), dtype, 0x200000)
    pt = FakeTensor((B, stride), torch.int32, 0x300000)
    lens = FakeTensor((B,), torch.int32, 0x400000)
    eight = dtype in (torch.float8_e4m3fn, torch.float8_e5m2)
    q = FakeTensor((B, R, Hq, d), torch.bfloat16 if eight else dtype, 0x500000)
    o = FakeTensor((B, R, Hq, d), q.dtype, 0x600000)
    return pa.make_io(q, o), pa.make_kv(k, v, pt, lens), pa.make_opts()


@pytest.fixture(scope="module")
def hctx(lib):
    return pa.attn_open_host_only(256)


def test_plan_headline_decode(hctx):
    io, kv, op = _decode_args(B=16, R=1, Hq=32, Hkv=8, d=128, stride=1024)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    # the VALU path with balanced partitions: equal lengths take one round of
    # 256 workgroups (one per CU: page tiles of 4 KiB), 32 per KV head, i.e. 2
    # partitions of 512 pages (8,192 tokens) per sequence at full capacity
    assert (P, T) == (2, 8192)
    # partial slots for up to two rounds (finer partitions for unequal lengths), 4 rows each
    assert W >= 1024 * 4 * (128 + 2) * 4


def test_plan_small_page_tiles_keep_two_workgroups_per_cu(hctx):
    # 8-bit K/V at d 128 (2 KiB page tiles): two workgroups per CU for equal
    # lengths, 64 per KV head -> 4 x 65,536 tokens in 16 partitions of 4,096
    io, kv, op = _decode_args(B=4, R=1, Hq=32, Hkv=8, d=128, stride=4096, dtype=torch.float8_e4m3fn)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert (P, T) == (16, 4096)


def test_plan_few_groups_fill_the_cus(hctx):
    # one KV head of the headline at R=8: 16 groups of 32 rows (the MFMA path at
    # one workgroup per CU) -> ranges of 1,024 tokens (32 per row), so 256
    # partial workgroups; a floor of 64 tokens per row would leave half idle
    io, kv, op = _decode_args(B=16, R=8, Hq=4, Hkv=1, d=128, stride=1024)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert (P, T) == (16, 1024) and 16 * P == 256


def test_plan_forced_splits(hctx):
    io, kv, op = _decode_args(stride=64)
    op.num_splits = 3
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert P == 3 and T * 3 >= 64 * 16


def test_plan_fp8_long_context(hctx):
    io, kv, op = _decode_args(B=4, R=4, Hq=32, Hkv=8, d=128, stride=4096, dtype=torch.float8_e4m3fn)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert 4 * 8 * P >= 256 and P * T >= 65536


def _status(fn):
    try:
        fn()
    except pa.AttnError as e:
        return e.status
    return pa.ATTN_OK


def test_host_only_context_never_enqueues(hctx):
    io, kv, op = _decode_args()
    ws = FakeTensor((1 << 24,), torch.uint8, 0x700000)
    assert _status(lambda: pa.attn_paged_decode(hctx, io, kv, op, ws, stream=0)) == pa.ATTN_ERR_DEVICE


@pytest.mark.parametrize("mutate,status", [
    (lambda io, kv, op: setattr(io, "q_rows", 9), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(io, "q_rows", 0), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(io, "num_q_heads", 7), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(io, "q", None), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(io, "q", 0x500008), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(kv, "k_pages", 0x100004), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(kv, "page_table", None), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(kv, "k_scale", 0.0), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(kv, "k_stride_head", 100), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(kv, "page_size", 32), pa.ATTN_ERR_UNSUPPORTED),
    (lambda io, kv, op: setattr(kv, "head_dim", 96), pa.ATTN_ERR_UNSUPPORTED),
    (lambda io, kv, op: setattr(io, "q_dtype", pa.ATTN_F16), pa.ATTN_ERR_UNSUPPORTED),
    (lambda io, kv, op: setattr(op, "block_mask", 0x800000), pa.ATTN_ERR_INVALID_ARGUMENT),
    (lambda io, kv, op: setattr(op, "num_splits", -1), pa.ATTN_ERR_INVALID_ARGUMENT),
    # rows addressing more than 2^30 tokens (int32 positions in the kernels)
    (lambda io, kv, op: setattr(kv, "page_table_stride", (1 << 26) + 1), pa.ATTN_ERR_UNSUPPORTED),
])
def test_decode_validation(hctx, mutate, status):
    io, kv, op = _decode_args()
    mutate(io, kv, op)
    ws = FakeTensor((1 << 24,), torch.uint8, 0x700000)
    assert _status(lambda: pa.attn_paged_decode(hctx, io, kv, op, ws, stream=0)) == status


def test_workspace_too_small(hctx):
    io, kv, op = _decode_args()
    _, _, need = pa.attn_paged_decode_plan(hctx, io, kv, op)
    ws = FakeTensor((need - 16,), torch.uint8, 0x700000)
    assert _status(lambda: pa.attn_paged_decode(hctx, io, kv, op, ws, stream=0)) == \
        pa.ATTN_ERR_WORKSPACE_TOO_SMALL


def _prefill_args(S=256, Hq=8, Hkv=2, d=64, dtype=torch.bfloat16, mask=False):
    io, kv, _ = _decode_args(B=1, R=S, Hq=Hq, Hkv=Hkv, d=d, stride=(S + 15) // 16, dtype=dtype)
    m = FakeTensor((1, 1, 2, 2), torch.uint8, 0x900000) if mask else None
    return io, kv, pa.make_opts(block_mask=m)


def test_prefill_validation(hctx):
    io, kv, op = _prefill_args()
    assert _status(lambda: pa.attn_prefill(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_DEVICE
    # a mask on the dense call, none on the sparse call
    io, kv, op = _prefill_args(mask=True)
    assert _status(lambda: pa.attn_prefill(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_INVALID_ARGUMENT
    assert _status(lambda: pa.attn_prefill_blocksparse(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_DEVICE
    op.mask_block = 100
    assert _status(lambda: pa.attn_prefill_blocksparse(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_INVALID_ARGUMENT
    op.mask_block, op.mask_heads = 128, 3
    assert _status(lambda: pa.attn_prefill_blocksparse(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_INVALID_ARGUMENT
    io, kv, op = _prefill_args()
    assert _status(lambda: pa.attn_prefill_blocksparse(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_INVALID_ARGUMENT
    # FP32 K/V prefill is not implemented
    io, kv, op = _prefill_args(dtype=torch.float32)
    assert _status(lambda: pa.attn_prefill(hctx, io, kv, op, stream=0)) == pa.ATTN_ERR_UNSUPPORTED


def test_read_probe_validation(hctx):
    buf = FakeTensor((1 << 20,), torch.uint8, 0x100000)
    order = FakeTensor((256,), torch.int32, 0x200000)
    sink = FakeTensor((1,), torch.int32, 0x300000)
    probe = lambda b, pat, o, s: _status(lambda: pa.attn_debug_read_probe(hctx, b, pat, o, s, stream=0))
    # valid requests validate, then a planning-only context enqueues nothing
    assert probe(buf, 0, None, sink) == pa.ATTN_ERR_DEVICE
    assert probe(buf, 1, order, sink) == pa.ATTN_ERR_DEVICE
    assert probe(buf, 2, order, sink) == pa.ATTN_ERR_DEVICE
    assert probe(buf, 3, order, sink) == pa.ATTN_ERR_INVALID_ARGUMENT           # no such pattern
    assert probe(buf, -1, order, sink) == pa.ATTN_ERR_INVALID_ARGUMENT
    assert probe(buf, 1, None, sink) == pa.ATTN_ERR_INVALID_ARGUMENT            # tiles need an order
    assert probe(buf, 2, None, sink) == pa.ATTN_ERR_INVALID_ARGUMENT
    assert probe(buf, 0, None, None) == pa.ATTN_ERR_INVALID_ARGUMENT            # no sink
    assert probe(FakeTensor((1000,), torch.uint8, 0x100000), 0, None, sink) == pa.ATTN_ERR_INVALID_ARGUMENT
    assert probe(FakeTensor((4096,), torch.uint8, 0x100004), 0, None, sink) == pa.ATTN_ERR_INVALID_ARGUMENT


def test_kv_append_validation(hctx):
    _, kv, _ = _decode_args(B=2, R=1, Hq=8, Hkv=2, d=64, stride=8)
    k = FakeTensor((2, 3, 2, 64), torch.bfloat16, 0x700000)
    v = FakeTensor((2, 3, 2, 64), torch.bfloat16, 0x800000)
    rows = pa.make_rows(k, v)
    app = lambda r: _status(lambda: pa.attn_kv_append(hctx, kv, r, stream=0))
    assert app(rows) == pa.ATTN_ERR_DEVICE                       # valid: nothing enqueued
    bad = pa.make_rows(k, v)
    bad.n_new = 0
    assert app(bad) == pa.ATTN_ERR_INVALID_ARGUMENT
    bad = pa.make_rows(k, v)
    bad.dtype = pa.ATTN_FP8_E4M3                                 # rows are F32/F16/BF16
    assert app(bad) == pa.ATTN_ERR_INVALID_ARGUMENT
    bad = pa.make_rows(k, v)
    bad.stride_row = 65                                          # 130 bytes: not 16-byte multiple
    assert app(bad) == pa.ATTN_ERR_INVALID_ARGUMENT
    bad = pa.make_rows(k, v)
    bad.v = 0x800008
    assert app(bad) == pa.ATTN_ERR_INVALID_ARGUMENT              # misaligned
    kv.k_scale = 0.0
    assert app(rows) == pa.ATTN_ERR_INVALID_ARGUMENT             # the scale divides


def test_head_dim_256_support(hctx):
    # decode: any rows (more than 8 per KV head run as blocks of 8); FP32 K/V only up to 128
    io, kv, op = _decode_args(B=2, R=8, Hq=16, Hkv=2, d=256, stride=64)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert P >= 1 and W > 0
    io, kv, op = _decode_args(B=2, R=1, Hq=8, Hkv=2, d=256, stride=64, dtype=torch.float32)
    assert _status(lambda: pa.attn_paged_decode_plan(hctx, io, kv, op)) == pa.ATTN_ERR_UNSUPPORTED
    # prefill at head_dim 256 validates (and a planning-only context enqueues nothing)
    q = FakeTensor((1, 64, 8, 256), torch.bfloat16, 0x500000)
    o = FakeTensor((1, 64, 8, 256), torch.bfloat16, 0x600000)
    k = FakeTensor((100, 2, 16, 256), torch.bfloat16, 0x100000)
    v = FakeTensor((100, 2, 256, 16), torch.bfloat16, 0x200000)
    pt = FakeTensor((1, 8), torch.int32, 0x300000)
    lens = FakeTensor((1,), torch.int32, 0x400000)
    kv = pa.make_kv(k, v, pt, lens)
    assert _status(lambda: pa.attn_prefill(hctx, pa.make_io(q, o), kv, pa.make_opts(), stream=0)) == \
        pa.ATTN_ERR_DEVICE
    # head_dim 96 is not built anywhere
    io, kv, op = _decode_args(d=96)
    assert _status(lambda: pa.attn_paged_decode_plan(hctx, io, kv, op)) == pa.ATTN_ERR_UNSUPPORTED


def _scales(pages=100, Hkv=2, ptr=0xA00000, strides=None):
    return FakeTensor((pages, Hkv, 16), torch.float32, ptr, strides)


@pytest.mark.parametrize("dtype", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_per_vector_scales_validate(hctx, dtype):
    io, _, op = _decode_args(dtype=dtype)
    k = FakeTensor((100, 2, 16, 128), dtype, 0x100000)
    v = FakeTensor((100, 2, 128, 16), dtype, 0x200000)
    pt = FakeTensor((2, 64), torch.int32, 0x300000)
    lens = FakeTensor((2,), torch.int32, 0x400000)
    ks, vs = _scales(ptr=0xA00000), _scales(ptr=0xB00000)
    kv = pa.make_kv(k, v, pt, lens, k_vscales=ks, v_vscales=vs)
    assert (kv.vscale_stride_page, kv.vscale_stride_head) == (32, 16)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert P >= 1 and W > 0
    plan = lambda kv: _status(lambda: pa.attn_paged_decode_plan(hctx, io, kv, op))
    kv.v_vscales = None                                           # both or neither
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = pa.make_kv(k, v, pt, lens, k_vscales=ks, v_vscales=vs)
    kv.k_vscales = 0xA00004                                       # misaligned
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = pa.make_kv(k, v, pt, lens, k_vscales=ks, v_vscales=vs)
    kv.vscale_stride_head = 8                                     # tiles overlap
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = pa.make_kv(k, v, pt, lens, k_vscales=ks, v_vscales=vs)
    kv.vscale_stride_page = 34                                    # not 16-byte aligned tiles
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    # per-vector scales belong to 8-bit storage only
    kb = FakeTensor((100, 2, 16, 128), torch.bfloat16, 0x100000)
    vb = FakeTensor((100, 2, 128, 16), torch.bfloat16, 0x200000)
    kv = pa.make_kv(kb, vb, pt, lens, k_vscales=ks, v_vscales=vs)
    iob, _, _ = _decode_args()
    assert _status(lambda: pa.attn_paged_decode_plan(hctx, iob, kv, op)) == pa.ATTN_ERR_INVALID_ARGUMENT
    # prefill validates the same way and then enqueues nothing on a planning-only context
    kv = pa.make_kv(k, v, pt, lens, k_vscales=ks, v_vscales=vs)
    q = FakeTensor((1, 256, 8, 128), torch.bfloat16, 0x500000)
    o = FakeTensor((1, 256, 8, 128), torch.bfloat16, 0x600000)
    assert _status(lambda: pa.attn_prefill(hctx, pa.make_io(q, o), kv, pa.make_opts(), stream=0)) == \
        pa.ATTN_ERR_DEVICE


def test_per_vector_append_needs_unit_tensor_scales(hctx):
    k = FakeTensor((100, 2, 16, 64), torch.float8_e5m2, 0x100000)
    v = FakeTensor((100, 2, 64, 16), torch.float8_e5m2, 0x200000)
    pt = FakeTensor((2, 8), torch.int32, 0x300000)
    lens = FakeTensor((2,), torch.int32, 0x400000)
    kv = pa.make_kv(k, v, pt, lens, k_vscales=_scales(), v_vscales=_scales(ptr=0xB00000))
    rows = pa.make_rows(FakeTensor((2, 3, 2, 64), torch.bfloat16, 0x700000),
                        FakeTensor((2, 3, 2, 64), torch.bfloat16, 0x800000))
    app = lambda: _status(lambda: pa.attn_kv_append(hctx, kv, rows, stream=0))
    assert app() == pa.ATTN_ERR_DEVICE                            # valid: nothing enqueued
    kv.v_scale = 2.0
    assert app() == pa.ATTN_ERR_INVALID_ARGUMENT


def test_fragment_tables_validate(hctx):
    io, _, op = _decode_args()
    kf = FakeTensor((8, 2, 16, 128), torch.bfloat16, 0x100000)       # one fragment of 8 pages
    vf = FakeTensor((8, 2, 128, 16), torch.bfloat16, 0x200000)
    pt = FakeTensor((2, 64), torch.int32, 0x300000)
    lens = FakeTensor((2,), torch.int32, 0x400000)
    tk = FakeTensor((13,), torch.int64, 0xC00000)
    tv = FakeTensor((13,), torch.int64, 0xD00000)
    mk = lambda **kw: pa.make_kv(kf, vf, pt, lens, k_fragments=tk, v_fragments=tv,
                                 fragment_pages_log2=3, num_pages=100, **kw)
    kv = mk()
    assert kv.k_pages is None and kv.num_pages == 100 and kv.num_fragments == 13
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert P >= 1
    plan = lambda kv: _status(lambda: pa.attn_paged_decode_plan(hctx, io, kv, op))
    kv = mk()
    kv.num_fragments = 12                                         # 12 x 8 < 100 pages
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = mk()
    kv.fragment_pages_log2 = 21
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = mk()
    kv.k_fragments = 0xC00004                                     # table misaligned
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    kv = mk()
    kv.k_fragments = None                                         # K then needs its pool
    assert plan(kv) == pa.ATTN_ERR_INVALID_ARGUMENT
    # the append and the gather take fragmented pools too
    rows = pa.make_rows(FakeTensor((2, 3, 2, 128), torch.bfloat16, 0x700000),
                        FakeTensor((2, 3, 2, 128), torch.bfloat16, 0x800000))
    assert _status(lambda: pa.attn_kv_append(hctx, mk(), rows, stream=0)) == pa.ATTN_ERR_DEVICE
    with pytest.raises(pa.AttnError):                             # a fragment view of 8 pages
        pa.make_kv(kf, vf, pt, lens, k_fragments=tk, v_fragments=tv, fragment_pages_log2=2,
                   num_pages=100)


def test_descriptors_keep_their_tensors_alive():
    """A descriptor holds raw pointers: the tensors it was made from must live as
    long as it does (else a caching allocator can hand their memory to the next
    allocation before the call runs)."""
    import gc
    import weakref
    k = torch.zeros((2, 3, 2, 64), dtype=torch.bfloat16)
    v = torch.zeros((2, 3, 2, 64), dtype=torch.bfloat16)
    wk, wv = weakref.ref(k), weakref.ref(v)
    rows = pa.make_rows(k, v)
    del k, v
    gc.collect()
    assert wk() is not None and wv() is not None
    del rows
    gc.collect()
    assert wk() is None and wv() is None


def test_capacity_at_the_limit_is_planned(hctx):
    io, kv, op = _decode_args(B=1, R=1, Hq=8, Hkv=2, d=128, stride=1 << 26)
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert P * T >= 1 << 30 and T <= 1 << 30


def test_noalloc_decode_validates_and_bounds_its_scratch(hctx):
    io, kv, op = _decode_args()
    assert _status(lambda: pa.attn_paged_decode_noalloc(hctx, io, kv, op, stream=0)) == \
        pa.ATTN_ERR_DEVICE
    io.q_rows = 9
    assert _status(lambda: pa.attn_paged_decode_noalloc(hctx, io, kv, op, stream=0)) == \
        pa.ATTN_ERR_INVALID_ARGUMENT
    # partials beyond the device-resident scratch: rejected before anything else
    io, kv, op = _decode_args(B=16, R=1, Hq=32, Hkv=8, d=128, stride=1024)
    op.num_splits = 128
    _, _, need = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    assert _status(lambda: pa.attn_paged_decode_noalloc(hctx, io, kv, op, stream=0)) == \
        pa.ATTN_ERR_WORKSPACE_TOO_SMALL


def test_plan_forced_splits_keep_partitions_per_sequence(hctx):
    # a forced split count keeps fixed partitions per (sequence, KV head)
    io, kv, op = _decode_args(B=16, R=1, Hq=32, Hkv=8, d=128, stride=1024)
    op.num_splits = 16
    P, T, W = pa.attn_paged_decode_plan(hctx, io, kv, op)
    assert (P, T) == (16, 1024) and W >= 16 * 8 * 4 * 16 * (128 + 2) * 4
