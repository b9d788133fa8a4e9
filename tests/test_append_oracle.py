"""Pins of the oracle's storage encoders and of its K/V append reference.

Each encoder is checked against what the number formats themselves fix
(every code round-trips, midpoints tie to the even code, overflow and NaN
behave as the formats define) and, where a library routine implements the
same rounding, against that routine (PyTorch's float32 -> bfloat16 / float16 /
float8_e4m3fn conversions, all round-to-nearest-even).  The append reference
is checked against the oracle's independent paged gather.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
import synth  # noqa: E402
from synth import DT_BF16, DT_BF8, DT_F16, DT_F32, DT_FP8  # noqa: E402


def _specials():
    f = np.float32
    v = [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-40, 2.0 ** -126, 2.0 ** -133, 2.0 ** -24,
         2.0 ** -25, 3 * 2.0 ** -26, 6e-8, 6.1e-5, 65504.0, 65519.0, 65520.0, 65536.0, 1e5,
         3.3895e38, 3.4e38, np.inf, -np.inf, np.nan, 448.0, 464.0, 465.0, 1e-3, -7.25]
    return np.array(v, dtype=f)


def _random(n, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal(n).astype(np.float32) * np.exp2(g.integers(-30, 30, n)).astype(np.float32)
    return x


def _torch_codes(x, dt, bits):
    return torch.from_numpy(x).to(dt).view(bits).numpy()


@pytest.mark.parametrize("dtype,tdt,bits", [(DT_BF16, torch.bfloat16, torch.int16),
                                            (DT_F16, torch.float16, torch.int16)])
def test_16bit_encoders_match_torch_rne(dtype, tdt, bits):
    x = np.concatenate([_specials(), _random(200000, 1)])
    got = oracle.encode(dtype, x)
    ref = _torch_codes(x, tdt, bits).astype(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (quiet, sign kept)
    dec = oracle.decode_codes(dtype, got[nan])
    assert np.all(np.isnan(dec))


@pytest.mark.parametrize("dtype", [DT_BF16, DT_F16])
def test_16bit_ties_go_to_even(dtype):
    # every pair of neighbouring positive codes: the midpoint takes the even code,
    # a hair above / below it takes the upper / lower code
    mb = 7 if dtype == DT_BF16 else 10
    top = 0x7F7F if dtype == DT_BF16 else 0x7BFF
    c = np.arange(1, top, 97, dtype=np.uint16)
    lo = oracle.decode_codes(dtype, c)
    hi = oracle.decode_codes(dtype, (c + 1).astype(np.uint16))
    mid = (lo + hi) / 2
    ok = mid == mid.astype(np.float32)                  # representable midpoints only
    mid32 = mid[ok].astype(np.float32)
    got = oracle.encode(dtype, mid32)
    even = np.where(c[ok] % 2 == 0, c[ok], c[ok] + 1)
    assert np.array_equal(got, even.astype(np.uint16))
    up = np.nextafter(mid32, np.float32(np.inf))
    dn = np.nextafter(mid32, np.float32(0))
    assert np.array_equal(oracle.encode(dtype, up), (c[ok] + 1).astype(np.uint16))
    assert np.array_equal(oracle.encode(dtype, dn), c[ok])
    assert mb > 0


def test_e4m3fn_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_codes(DT_FP8, codes).astype(np.float32)
    got = oracle.encode(DT_FP8, vals)
    finite = ~np.isnan(vals)
    assert np.array_equal(got[finite], codes[finite])
    assert set(got[~finite].tolist()) <= {0x7F, 0xFF}


def test_e4m3fn_ties_saturation_and_nan():
    codes = np.arange(0, 0x7E, dtype=np.uint8)                  # 0 .. 416 (0x7D)
    lo = oracle.decode_codes(DT_FP8, codes)
    hi = oracle.decode_codes(DT_FP8, codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)                    # exact: <= 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(oracle.encode(DT_FP8, mid), even)
    assert np.array_equal(oracle.encode(DT_FP8, np.nextafter(mid, np.float32(np.inf))), codes + 1)
    assert np.array_equal(oracle.encode(DT_FP8, -mid), even | 0x80)
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, np.inf], dtype=np.float32)
    assert np.all(oracle.encode(DT_FP8, big) == 0x7E)
    assert np.all(oracle.encode(DT_FP8, -big) == 0xFE)
    assert oracle.encode(DT_FP8, np.array([np.nan], np.float32))[0] in (0x7F, 0xFF)
    # subnormals are multiples of 2^-9; half of the smallest one ties to zero
    assert oracle.encode(DT_FP8, np.array([2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9], np.float32)).tolist() == [0, 2, 1]


def test_e4m3fn_matches_torch_in_range():
    x = _random(200000, 2)
    x = x[np.abs(x) < 448.0]
    got = oracle.encode(DT_FP8, x)
    ref = _torch_codes(x, torch.float8_e4m3fn, torch.uint8)
    assert np.array_equal(got, ref)


def test_e5m2_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_codes(DT_BF8, codes).astype(np.float32)
    got = oracle.encode(DT_BF8, vals)
    finite = ~np.isnan(vals)
    assert np.array_equal(got[finite], codes[finite])          # infinities included
    assert set(got[~finite].tolist()) <= {0x7F, 0xFF}


def test_e5m2_ties_saturation_and_specials():
    codes = np.arange(0, 0x7B, dtype=np.uint8)                  # 0 .. 49152 (0x7A)
    lo = oracle.decode_codes(DT_BF8, codes)
    hi = oracle.decode_codes(DT_BF8, codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)                    # exact: <= 4 significant bits
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(oracle.encode(DT_BF8, mid), even)
    assert np.array_equal(oracle.encode(DT_BF8, np.nextafter(mid, np.float32(np.inf))), codes + 1)
    assert np.array_equal(oracle.encode(DT_BF8, np.nextafter(mid, np.float32(0))), codes)
    assert np.array_equal(oracle.encode(DT_BF8, -mid), even | 0x80)
    big = np.array([57344.0, 57345.0, 61439.0, 61440.0, 1e6, 3e38], dtype=np.float32)
    assert np.all(oracle.encode(DT_BF8, big) == 0x7B)           # finite: saturate
    assert np.all(oracle.encode(DT_BF8, -big) == 0xFB)
    inf = np.array([np.inf, -np.inf], dtype=np.float32)
    assert oracle.encode(DT_BF8, inf).tolist() == [0x7C, 0xFC]   # infinities stay
    assert oracle.encode(DT_BF8, np.array([np.nan], np.float32))[0] in (0x7F, 0xFF)
    # subnormals are multiples of 2^-16; half of the smallest one ties to zero
    assert oracle.encode(DT_BF8, np.array([2.0 ** -17, 3 * 2.0 ** -17, 2.0 ** -16], np.float32)).tolist() == [0, 2, 1]


def test_e5m2_matches_torch_in_range():
    x = _random(200000, 5)
    x = x[np.abs(x) < 57344.0]
    got = oracle.encode(DT_BF8, x)
    ref = _torch_codes(x, torch.float8_e5m2, torch.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype,fmax", [(DT_FP8, 448.0), (DT_BF8, 57344.0)])
def test_vector_scales_rule(dtype, fmax):
    g = np.random.default_rng(6)
    x = (g.standard_normal((300, 64)) * np.exp2(g.integers(-20, 20, (300, 1)))).astype(np.float32)
    x[0] = 0.0                                                  # all zero: scale 1
    x[1, :] = 0.0
    x[1, 5] = np.inf                                            # non-finite entries do not count
    x[1, 6] = np.nan
    x[1, 7] = -3.0
    x[2, :] = 1e-44                                             # quotient underflows to 0: scale 1
    sc = oracle.vector_scales(dtype, x)
    amax = np.array([np.max(np.abs(r[np.isfinite(r)]), initial=0.0) for r in x], dtype=np.float32)
    ref = (amax / np.float32(fmax)).astype(np.float32)
    ref = np.where(ref == 0, np.float32(1.0), ref)
    assert np.array_equal(sc, ref)
    assert sc[0] == 1.0 and sc[2] == 1.0 and sc[1] == np.float32(3.0) / np.float32(fmax)
    # codes: one single-precision division by the vector's own scale
    codes = oracle.encode_vectors(dtype, x, sc)
    q = (x / sc[:, None]).astype(np.float32)
    assert np.array_equal(codes, oracle.encode(dtype, q))
    # the largest finite magnitude of each ordinary vector lands on the largest code
    big = np.abs(codes[3:].astype(np.int32) & 0x7F).max(axis=1)
    assert np.all(big == (0x7E if dtype == DT_FP8 else 0x7B))
    # and the dequantised vector is within half a grid step (relative 2^-(m+1)) of x
    mb = 3 if dtype == DT_FP8 else 2
    xh = oracle.decode_codes(dtype, codes[3:]).reshape(-1, 64) * sc[3:, None]
    rel_ok = np.abs(xh - x[3:]) <= np.abs(x[3:]) * 2.0 ** -(mb + 1) + sc[3:, None] * 2.0 ** -(16 if dtype == DT_BF8 else 9)
    assert np.all(rel_ok)


@pytest.mark.parametrize("dtype", [DT_F32, DT_F16, DT_BF16, DT_FP8])
def test_scale_is_one_single_precision_division(dtype):
    x = _random(50000, 3)
    s = np.float32(0.0123456)
    q = (x / s).astype(np.float32)           # numpy float32 division: IEEE, correctly rounded
    assert np.array_equal(oracle.encode(dtype, x, s), oracle.encode(dtype, q, 1.0))


@pytest.mark.parametrize("kv_dtype", [DT_FP8, DT_BF8])
def test_per_vector_append_lands_where_the_gather_reads(kv_dtype):
    lens = [37, 5, 16, 64]
    n_new = 7
    p = synth.make_decode(52, 4, 4, 2, 64, lens, 1, kv_dtype=kv_dtype, stride=5, vscales=True)
    kcodes, vcodes = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    kvs, vvs = p.k_vs.numpy(), p.v_vs.numpy()
    g = np.random.default_rng(7)
    knew = (g.standard_normal((4, n_new, 2, 64)) * 3).astype(np.float32)
    vnew = (g.standard_normal((4, n_new, 2, 64)) / 5).astype(np.float32)
    pt = p.page_table.numpy()
    kout, vout, kvs2, vvs2 = oracle.kv_append(kv_dtype, kcodes, vcodes, pt, p.seq_lens.numpy(),
                                              knew, vnew, k_vs=kvs, v_vs=vvs)
    p2 = synth.with_pool_codes(p, kout, vout)
    p2.k_vs, p2.v_vs = torch.from_numpy(kvs2), torch.from_numpy(vvs2)
    for b, L in enumerate(lens):
        for gg in range(2):
            k_old, v_old = oracle.gather(p, b, gg)
            k_new, v_new = oracle.gather(p2, b, gg)
            for pos in range(L):
                i = pos - (L - n_new)
                if i < 0:
                    assert np.array_equal(k_new[pos], k_old[pos]) and np.array_equal(v_new[pos], v_old[pos])
                    continue
                for src, got in ((knew[b, i, gg], k_new[pos]), (vnew[b, i, gg], v_new[pos])):
                    amax = np.float32(np.abs(src).max())
                    u = np.float32(amax / np.float32(oracle.FMAX[kv_dtype]))
                    exp = oracle.decode_codes(kv_dtype, oracle.encode(kv_dtype, src, u)) * np.float64(u)
                    assert np.array_equal(got, exp)
    # only the new slots' scales changed (NaN pad scales compare as unchanged)
    same = lambda a, b: (a == b) | (np.isnan(a) & np.isnan(b))
    for new, old in ((kvs2, kvs), (vvs2, vvs)):
        assert int((~same(new, old)).sum()) <= sum(min(L, n_new) for L in lens) * 2


@pytest.mark.parametrize("kv_dtype", [DT_F32, DT_BF16, DT_FP8, DT_BF8])
def test_append_reference_lands_where_the_gather_reads(kv_dtype):
    # sequences of different lengths, n_new rows each; one sequence shorter
    # than n_new (its first rows are dropped)
    lens = [37, 5, 16, 64]
    n_new = 7
    p = synth.make_decode(51, 4, 4, 2, 64, lens, 1, kv_dtype=kv_dtype, stride=5)
    kcodes = synth.pool_codes(p.k_pool)
    vcodes = synth.pool_codes(p.v_pool)
    g = np.random.default_rng(4)
    knew = g.standard_normal((4, n_new, 2, 64)).astype(np.float32)
    vnew = g.standard_normal((4, n_new, 2, 64)).astype(np.float32)
    pt = p.page_table.numpy()
    kout, vout = oracle.kv_append(kv_dtype, kcodes, vcodes, pt, p.seq_lens.numpy(), knew, vnew,
                                  p.k_scale, p.v_scale)
    p2 = synth.with_pool_codes(p, kout, vout)
    for b, L in enumerate(lens):
        for gg in range(2):
            k_old, v_old = oracle.gather(p, b, gg)
            k_new, v_new = oracle.gather(p2, b, gg)
            for pos in range(L):
                i = pos - (L - n_new)
                if i < 0:       # untouched rows
                    assert np.array_equal(k_new[pos], k_old[pos]) and np.array_equal(v_new[pos], v_old[pos])
                else:
                    kexp = oracle.decode_codes(kv_dtype, oracle.encode(kv_dtype, knew[b, i, gg], p.k_scale)) * p.k_scale
                    vexp = oracle.decode_codes(kv_dtype, oracle.encode(kv_dtype, vnew[b, i, gg], p.v_scale)) * p.v_scale
                    assert np.array_equal(k_new[pos], kexp) and np.array_equal(v_new[pos], vexp)
    # nothing outside those slots changed: count the changed K codes
    changed = int((kout != kcodes).any(axis=-1).sum())
    expected = sum(min(L, n_new) for L in lens) * 2
    assert changed <= expected


@pytest.mark.parametrize("kv_dtype", [DT_BF16, DT_FP8])
def test_append_reference_clamps_lengths_to_the_capacity(kv_dtype):
    """seq_lens above the page table's capacity: the new rows land at the last
    positions the table addresses, as the (independently pinned) gather reads
    them back; earlier rows stay as they were."""
    stride, n_new = 3, 5
    cap = stride * 16
    p = synth.make_decode(52, 2, 4, 2, 64, [cap, cap], 1, kv_dtype=kv_dtype, stride=stride)
    kcodes, vcodes = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    g = np.random.default_rng(5)
    knew = g.standard_normal((2, n_new, 2, 64)).astype(np.float32)
    vnew = g.standard_normal((2, n_new, 2, 64)).astype(np.float32)
    lens_call = np.array([cap + 3, 2 ** 30], dtype=np.int32)
    kout, vout = oracle.kv_append(kv_dtype, kcodes, vcodes, p.page_table.numpy(), lens_call,
                                  knew, vnew, p.k_scale, p.v_scale)
    p2 = synth.with_pool_codes(p, kout, vout)
    for b in range(2):
        for gg in range(2):
            k_old, v_old = oracle.gather(p, b, gg)
            k_new, v_new = oracle.gather(p2, b, gg)
            assert np.array_equal(k_new[:cap - n_new], k_old[:cap - n_new])
            assert np.array_equal(v_new[:cap - n_new], v_old[:cap - n_new])
            for i in range(n_new):
                kexp = oracle.decode_codes(kv_dtype, oracle.encode(kv_dtype, knew[b, i, gg], p.k_scale)) * p.k_scale
                vexp = oracle.decode_codes(kv_dtype, oracle.encode(kv_dtype, vnew[b, i, gg], p.v_scale)) * p.v_scale
                assert np.array_equal(k_new[cap - n_new + i], kexp)
                assert np.array_equal(v_new[cap - n_new + i], vexp)
