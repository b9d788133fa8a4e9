"""GPU parity of the K/V append (attn_kv_append): the pools after the call
must equal, byte for byte, the oracle's append reference (integer and byte
work: bit-exact), for every storage type and source type; and attention over
the appended cache must match the oracle over the expected cache."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
import paged_gqa_attention_amd as pa  # noqa: E402
import synth  # noqa: E402
from synth import DT_BF16, DT_BF8, DT_F16, DT_F32, DT_FP8  # noqa: E402
from helpers import Dev, check_full, ctx, run  # noqa: E402

pytestmark = pytest.mark.gpu

SRC = {DT_F32: torch.float32, DT_F16: torch.float16, DT_BF16: torch.bfloat16}


def _say(*a):
    print("[append]", *a, flush=True)


def _inject_specials(k: torch.Tensor, seed: int):
    """Overwrite a few source values with NaN, +-inf, huge, tiny and exact ties."""
    flat = k.view(-1)
    g = torch.Generator().manual_seed(seed)
    idx = torch.randperm(flat.numel(), generator=g)[:64]
    vals = torch.tensor([float("nan"), float("inf"), -float("inf"), 1e30, -1e30, 1e-30, 3e-5,
                         -2.0 ** -10, 1.0625, 65520.0, 448.0, 464.0] * 6, dtype=torch.float32)
    flat[idx] = vals[: idx.numel()].to(flat.dtype)


def _append_case(seed, kv_dtype, src_dtype, d, lens, n_new, stride, specials=False, hkv=2,
                 lens_after=None):
    p = synth.make_decode(seed, len(lens), 4 * hkv, hkv, d, lens, 1, kv_dtype=kv_dtype,
                          stride=stride)
    if lens_after is not None:     # seq_lens as the caller passes them (may exceed capacity)
        p.seq_lens = torch.tensor(lens_after, dtype=torch.int32)
    knew, vnew = synth.append_rows(seed + 1, len(lens), n_new, hkv, d, dtype=SRC[src_dtype])
    if specials:
        _inject_specials(knew, seed)
        _inject_specials(vnew, seed + 7)
    k0, v0 = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    kexp, vexp = oracle.kv_append(kv_dtype, k0, v0, p.page_table.numpy(), p.seq_lens.numpy(),
                                  knew.float().numpy(), vnew.float().numpy(), p.k_scale, p.v_scale)
    dev = Dev(p)
    _say(f"seed={seed} kv={kv_dtype} src={src_dtype} d={d} lens={lens} n_new={n_new}")
    kv = pa.make_kv(dev.k, dev.v, dev.pt, dev.lens, p.k_scale, p.v_scale)
    pa.attn_kv_append(ctx(), kv, pa.make_rows(knew.cuda(), vnew.cuda()))
    torch.cuda.synchronize()
    kgot, vgot = synth.pool_codes(dev.k), synth.pool_codes(dev.v)
    return p, dev, (kgot, vgot), (kexp, vexp)


def _same_codes(kv_dtype, got, exp):
    if kv_dtype == DT_F32:      # NaN payloads of a division are not specified: both NaN
        g, e = got.view(np.float32), exp.view(np.float32)
        nan = np.isnan(e)
        return np.array_equal(np.isnan(g), nan) and np.array_equal(got[~nan], exp[~nan])
    return np.array_equal(got, exp)


@pytest.mark.parametrize("kv_dtype", [DT_F32, DT_F16, DT_BF16, DT_FP8])
@pytest.mark.parametrize("src_dtype", [DT_F32, DT_F16, DT_BF16])
def test_append_bit_exact(kv_dtype, src_dtype):
    # ragged lengths: mid-page starts, a sequence shorter than n_new, page-aligned ends
    _, _, got, exp = _append_case(600 + 10 * kv_dtype + src_dtype, kv_dtype, src_dtype, 64,
                                  [37, 5, 16, 64, 300], 23, 20)
    for gt, ex in zip(got, exp):
        assert _same_codes(kv_dtype, gt, ex)


@pytest.mark.parametrize("kv_dtype", [DT_F32, DT_F16, DT_BF16, DT_FP8])
@pytest.mark.parametrize("src_dtype", [DT_F32, DT_F16, DT_BF16])
@pytest.mark.parametrize("n_new,d", [(1, 64), (3, 128), (8, 64), (2, 256)])
def test_append_few_rows_bit_exact(kv_dtype, src_dtype, n_new, d):
    """Decode and verify steps (at most 8 new rows per sequence take the one-wave
    path): mid-page and page-aligned ends, a sequence shorter than n_new, special
    values."""
    _, _, got, exp = _append_case(750 + 10 * kv_dtype + src_dtype + 100 * n_new, kv_dtype,
                                  src_dtype, d, [37, 2, 16, 64, 300], n_new, 20, specials=True)
    for gt, ex in zip(got, exp):
        assert _same_codes(kv_dtype, gt, ex)


@pytest.mark.parametrize("kv_dtype", [DT_F16, DT_BF16, DT_FP8, DT_F32])
def test_append_special_values(kv_dtype):
    _, _, got, exp = _append_case(700 + kv_dtype, kv_dtype, DT_F32, 128, [40, 129], 40, 9,
                                  specials=True)
    for gt, ex in zip(got, exp):
        assert _same_codes(kv_dtype, gt, ex)


@pytest.mark.parametrize("n_new", [1, 16, 300])
def test_append_d128_decode_and_prefill_shapes(n_new):
    # one row per sequence (a decode step), a page, a prefill chunk
    _, _, got, exp = _append_case(710 + n_new, DT_BF16, DT_BF16, 128, [1000, 301, 17, 2048], n_new, 128)
    for gt, ex in zip(got, exp):
        assert np.array_equal(gt, ex)


def test_append_clamps_to_capacity():
    # seq_lens beyond the table's capacity: rows land at the capacity's end
    _, _, got, exp = _append_case(720, DT_BF16, DT_F32, 64, [64, 64], 10, 4, lens_after=[100, 64])
    for gt, ex in zip(got, exp):
        assert np.array_equal(gt, ex)


@pytest.mark.parametrize("kv_dtype", [DT_BF16, DT_FP8])
def test_attention_over_the_appended_cache(kv_dtype):
    """Append 4 verify rows' K/V, then decode those 4 rows: the result equals the
    oracle's attention over the expected cache."""
    p, dev, got, exp = _append_case(730 + kv_dtype, kv_dtype, DT_BF16, 128, [700, 1500, 33], 4, 128)
    assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1])
    p.q_rows = 4
    p.q = synth.normal(731, 0, (3, 4, 8, 128)).to(p.q.dtype)
    dev.q = p.q.cuda()
    o, lse = run(dev)
    pexp = synth.with_pool_codes(p, exp[0], exp[1])
    check_full(pexp, o, lse)


@pytest.mark.parametrize("kv_dtype", [DT_BF16, DT_FP8])
def test_append_head_dim_256(kv_dtype):
    _, _, got, exp = _append_case(740 + kv_dtype, kv_dtype, DT_F32, 256, [70, 300, 16], 37, 24)
    for gt, ex in zip(got, exp):
        assert np.array_equal(gt, ex)


def _encoder_probe_values(kv_dtype) -> np.ndarray:
    """Every finite code value of the format, the midpoints between neighbours
    (ties, which go to the even code), the midpoints one FP32 ulp either side,
    values past the largest finite code, infinities, NaN, zeros and FP32
    denormals, with both signs."""
    t = torch.float8_e4m3fn if kv_dtype == DT_FP8 else torch.float8_e5m2
    v = torch.arange(256, dtype=torch.uint8).view(t).to(torch.float64).numpy()
    v = np.unique(v[np.isfinite(v) & (v >= 0)])
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    big = np.float32(v[-1])
    extra = np.array([big * 1.01, big * 1.0625, big * 1.125, big * 1.2, 1e30, np.inf, np.nan,
                      1e-40, 1e-45, 0.0], dtype=np.float32)
    pos = np.concatenate([v.astype(np.float32), mids, up, dn, extra])
    return np.concatenate([pos, -pos]).astype(np.float32)


@pytest.mark.parametrize("kv_dtype", [DT_FP8, DT_BF8])
def test_append_encoder_dense(kv_dtype):
    """The 8-bit encoders against the oracle's, bit for bit, on every code
    value, every tie and its neighbours (unit scales, FP32 source rows)."""
    _say("encoder dense", kv_dtype)
    vals = _encoder_probe_values(kv_dtype)
    B, n_new, hkv, d = 2, 24, 2, 64
    slots = B * n_new * hkv * d
    assert vals.size <= slots
    g = np.random.default_rng(kv_dtype)
    kf = np.resize(vals, slots)
    vf = np.resize(vals[g.permutation(vals.size)], slots)
    knew = torch.from_numpy(kf.reshape(B, n_new, hkv, d).copy())
    vnew = torch.from_numpy(vf.reshape(B, n_new, hkv, d).copy())
    p = synth.make_decode(750 + kv_dtype, B, 4 * hkv, hkv, d, [40, 24], 1, kv_dtype=kv_dtype,
                          stride=5)
    k0, v0 = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    kexp, vexp = oracle.kv_append(kv_dtype, k0, v0, p.page_table.numpy(), p.seq_lens.numpy(),
                                  knew.numpy(), vnew.numpy(), 1.0, 1.0)
    dev = Dev(p)
    kv = pa.make_kv(dev.k, dev.v, dev.pt, dev.lens, 1.0, 1.0)
    pa.attn_kv_append(ctx(), kv, pa.make_rows(knew.cuda(), vnew.cuda()))
    torch.cuda.synchronize()
    assert np.array_equal(synth.pool_codes(dev.k), kexp)
    assert np.array_equal(synth.pool_codes(dev.v), vexp)
