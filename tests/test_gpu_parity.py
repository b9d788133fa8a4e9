"""GPU parity: the HIP path through the C ABI against the FP64 oracle, element
by element, at sizes that span several tiles/partitions and ragged tails,
plus the invariants the pages state (page permutation, split + merge,
all-ones mask, sink = -inf, replay determinism)."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_amd as pa
import synth
from synth import DT_BF16, DT_BF8, DT_F16, DT_F32, DT_FP8

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, ctx, run  # noqa: E402


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ gather / codecs

@pytest.mark.parametrize("dtype", [DT_F32, DT_F16, DT_BF16, DT_FP8])
def test_debug_gather_bit_exact(dtype):
    _say("gather", dtype)
    p = synth.make_decode(61, 2, 4, 2, 64, [70, 33], 1, kv_dtype=dtype, stride=8, extra_pages=3)
    d = Dev(p)
    for b in range(2):
        L = int(p.seq_lens[b])
        ko = torch.empty((2, L, 64), dtype=torch.float32, device="cuda")
        vo = torch.empty_like(ko)
        kv = pa.make_kv(d.k, d.v, d.pt, d.lens, p.k_scale, p.v_scale)
        pa.attn_debug_gather_kv(ctx(), kv, b, L, ko, vo)
        torch.cuda.synchronize()
        for g in range(2):
            k, v = oracle.gather(p, b, g)
            # FP32 products of exact codes and FP32 scales are exact in FP64
            assert np.array_equal(ko[g].double().cpu().numpy(), k.astype(np.float32).astype(np.float64)) or \
                np.array_equal(ko[g].double().cpu().numpy(), k)
            assert np.array_equal(vo[g].double().cpu().numpy(), v.astype(np.float32).astype(np.float64)) or \
                np.array_equal(vo[g].double().cpu().numpy(), v)


def test_fp8_every_code_decodes_exactly():
    """All 256 e4m3fn codes through the kernels' FP32 and 16-bit conversions."""
    _say("fp8 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    k = codes.view(1, 1, 16, 16).repeat(1, 1, 1, 4).contiguous()   # 1 page, d=64
    k = k.view(torch.float8_e4m3fn)
    v = k.transpose(2, 3).contiguous()
    pt = torch.zeros((1, 1), dtype=torch.int32)
    lens = torch.tensor([16], dtype=torch.int32)
    kd, vd, ptd, ld = k.cuda(), v.cuda(), pt.cuda(), lens.cuda()
    kv = pa.make_kv(kd, vd, ptd, ld)
    ko = torch.empty((1, 16, 64), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    pa.attn_debug_gather_kv(ctx(), kv, 0, 16, ko, vo)
    torch.cuda.synchronize()
    ref = oracle.decode_codes(DT_FP8, k.view(torch.uint8).numpy().reshape(-1)).reshape(16, 64)
    got = ko[0].double().cpu().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------------ decode

DECODE_CASES = [
    # (name, kwargs)
    ("cfg1", dict(fn="config1")),
    ("bf16_r1_g4", dict(B=3, Hq=32, Hkv=8, d=128, lens=[1000, 37, 2100], R=1, dt=DT_BF16)),
    ("bf16_r4_g4", dict(B=3, Hq=32, Hkv=8, d=128, lens=[1000, 37, 2100], R=4, dt=DT_BF16)),
    ("bf16_r8_g4", dict(B=3, Hq=32, Hkv=8, d=128, lens=[1000, 37, 2100], R=8, dt=DT_BF16)),
    ("bf16_r2_g4_sink", dict(B=2, Hq=8, Hkv=2, d=128, lens=[515, 1700], R=2, dt=DT_BF16, sinks=True)),
    ("f16_r1_d64", dict(B=2, Hq=8, Hkv=2, d=64, lens=[300, 1029], R=1, dt=DT_F16)),
    ("f16_r8_d64", dict(B=2, Hq=8, Hkv=2, d=64, lens=[300, 1029], R=8, dt=DT_F16, sinks=True)),
    ("fp8_r4", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=4, dt=DT_FP8)),
    ("fp8_r1", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=1, dt=DT_FP8, sinks=True)),
    ("fp8_r8_d64_f16q", dict(B=2, Hq=16, Hkv=2, d=64, lens=[600, 90], R=8, dt=DT_FP8, q=DT_F16)),
    ("f32_r1_d128", dict(B=2, Hq=8, Hkv=2, d=128, lens=[300, 700], R=1, dt=DT_F32, o=DT_F32)),
    ("f32_r4_g4", dict(B=2, Hq=8, Hkv=2, d=64, lens=[300, 700], R=4, dt=DT_F32, o=DT_F32, sinks=True)),
    ("f32_q_bf16", dict(B=1, Hq=4, Hkv=1, d=64, lens=[500], R=3, dt=DT_F32, q=DT_BF16, o=DT_F32)),
    ("mha_r8", dict(B=2, Hq=4, Hkv=4, d=128, lens=[200, 400], R=8, dt=DT_BF16)),
    ("g8_r8_64rows", dict(B=1, Hq=16, Hkv=2, d=128, lens=[1100], R=8, dt=DT_BF16)),
    ("g3_r5_odd", dict(B=2, Hq=6, Hkv=2, d=64, lens=[77, 130], R=5, dt=DT_BF16, sinks=True)),
    ("empty_and_short", dict(B=3, Hq=8, Hkv=2, d=128, lens=[0, 3, 50], R=4, dt=DT_BF16, sinks=True)),
    ("empty_no_sink", dict(B=2, Hq=8, Hkv=2, d=64, lens=[0, 20], R=1, dt=DT_BF16)),
    ("fp32_out_bf16_kv", dict(B=2, Hq=8, Hkv=2, d=128, lens=[400, 90], R=4, dt=DT_BF16, o=DT_F32)),
]


def _decode_problem(kw, seed=0):
    if kw.get("fn") == "config1":
        return synth.config1()
    return synth.make_decode(seed or 71, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["lens"], kw["R"],
                             kv_dtype=kw["dt"], q_dtype=kw.get("q"), o_dtype=kw.get("o"),
                             sinks=kw.get("sinks", False), stride=kw.get("stride"))


@pytest.mark.parametrize("name,kw", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(name, kw):
    _say("decode", name)
    p = _decode_problem(kw)
    d = Dev(p)
    o, l = run(d)
    check_full(p, o, l, label=name)


@pytest.mark.parametrize("splits", [1, 2, 5, 64])
def test_decode_forced_splits(splits):
    """Any partition count gives the unsplit result within FP32 rounding
    (Geramy/LSE releases, v0.4.20: split and unsplit responses identical)."""
    _say("splits", splits)
    p = synth.make_decode(72, 2, 8, 2, 128, [2000, 513], 4, kv_dtype=DT_BF16, o_dtype=DT_F32,
                          sinks=True)
    d = Dev(p)
    o, l = run(d, num_splits=splits)
    check_full(p, o, l, tol=2e-3, label=f"splits={splits}")


SHORT_IN_LONG = [
    ("valu_r1_bf16", 1, 128, 32, 8, DT_BF16),
    ("valu_r2_f16_d64", 2, 64, 8, 2, DT_F16),
    ("valu_r1_fp8", 1, 128, 32, 8, DT_FP8),
    ("mfma_r4_bf16", 4, 128, 32, 8, DT_BF16),
    ("mfma_r8_fp8", 8, 128, 16, 4, DT_FP8),
    ("wide_r4_d256", 4, 256, 16, 4, DT_BF16),
    ("valu_r1_d256", 1, 256, 8, 2, DT_BF16),
]


@pytest.mark.parametrize("name,R,d,Hq,Hkv,dt", SHORT_IN_LONG, ids=[c[0] for c in SHORT_IN_LONG])
def test_decode_short_sequences_in_long_tables(name, R, d, Hq, Hkv, dt):
    """Sequences far shorter than the page table's capacity (65,536 tokens): the
    kernels size their partitions from the longest sequence of the call, so the
    partition boundaries differ from the plan's; the result must not."""
    _say("short in long", name)
    p = synth.make_decode(231, 4, Hq, Hkv, d, [2500, 100, 7, 1999], R, kv_dtype=dt,
                          stride=4096, sinks=True)
    o, l = run(Dev(p))
    check_full(p, o, l, label=name)


@pytest.mark.parametrize("R", [1, 4])
def test_decode_many_sequences_short_in_long_tables(R):
    """More than 64 sequences (the kernels then find the longest with vector
    loads and a reduction across the wave), far shorter than the capacity."""
    _say("many short in long", R)
    lens = [int(x) for x in (np.arange(80) * 37 % 611 + 1)]
    p = synth.make_decode(232, 80, 8, 2, 64, lens, R, kv_dtype=DT_BF16, stride=256, sinks=True)
    o, l = run(Dev(p))
    check_full(p, o, l, label=f"B=80 R={R}")


@pytest.mark.parametrize("dt,R", [(DT_BF16, 1), (DT_F16, 2), (DT_FP8, 1), (DT_BF16, 4), (DT_FP8, 8)])
def test_decode_partition_longer_than_8192_tokens(dt, R):
    """One partition of 20,480 tokens (forced): a wave of the VALU kernel (R <= 2)
    walks 320 pages, its page ids loaded in three blocks of 128; a wave of the
    MFMA kernel (R = 4, 8) walks 160 page pairs, their ids in three blocks of 64."""
    _say("long partition", dt, R)
    p = synth.make_decode(233, 2, 8, 2, 64, [20000, 9000], R, kv_dtype=dt, stride=1280,
                          sinks=True)
    o, l = run(Dev(p), num_splits=1)
    check_full(p, o, l, label=f"dt={dt} R={R}")


def test_decode_page_permutation_bit_identical():
    _say("decode permutation")
    p = synth.make_decode(73, 2, 32, 8, 128, [900, 1333], 4, kv_dtype=DT_BF16, extra_pages=7)
    o0, l0 = run(Dev(p))
    perm = synth.permutation(73, 9, p.num_pages)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(p.num_pages)
    p.k_pool = p.k_pool[inv].contiguous()
    p.v_pool = p.v_pool[inv].contiguous()
    p.page_table = perm[p.page_table.long()].to(torch.int32)
    o1, l1 = run(Dev(p))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_decode_sink_minus_inf_bit_identical():
    _say("decode sink -inf")
    p = synth.make_decode(74, 2, 8, 2, 128, [400, 800], 1, kv_dtype=DT_BF16)
    o0, l0 = run(Dev(p))
    p.sinks = torch.full((8,), -math.inf, dtype=torch.float32)
    o1, l1 = run(Dev(p))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_decode_replay_deterministic():
    _say("decode replay")
    p = synth.make_decode(75, 3, 32, 8, 128, [3000, 100, 2000], 8, kv_dtype=DT_BF16, sinks=True)
    d = Dev(p)
    o0, l0 = run(d)
    o1, l1 = run(d)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_decode_verify_row_matches_single_row_decode():
    """Verify row r equals an R=1 decode at length L - R + r + 1 (within rounding)."""
    _say("verify rows")
    R = 8
    p = synth.make_decode(76, 1, 32, 8, 128, [1000], R, kv_dtype=DT_BF16, o_dtype=DT_F32)
    o, _ = run(Dev(p))
    for r in [0, 3, 7]:
        q1 = synth.make_decode(76, 1, 32, 8, 128, [1000], 1, kv_dtype=DT_BF16, o_dtype=DT_F32)
        q1.k_pool, q1.v_pool, q1.page_table = p.k_pool, p.v_pool, p.page_table
        q1.seq_lens = torch.tensor([1000 - R + r + 1], dtype=torch.int32)
        q1.q = p.q[:, r:r + 1].clone()
        o1, _ = run(Dev(q1))
        assert np.max(np.abs(o1[0, 0] - o[0, r])) <= 2e-3


def test_decode_buffers_untouched_outside_outputs():
    """Guard bands around O stay intact and inputs are not modified."""
    _say("decode guards")
    p = synth.make_decode(77, 2, 8, 2, 128, [300, 600], 4, kv_dtype=DT_BF16)
    d = Dev(p)
    big = torch.full((3, 2, 4, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o = big[1]
    before = [t.clone() for t in (d.q, d.k, d.v, d.pt, d.lens)]
    pa.paged_decode(ctx(), d.q, d.k, d.v, d.pt, d.lens, out=o)
    torch.cuda.synchronize()
    assert torch.all(big[0] == 7.0) and torch.all(big[2] == 7.0)
    for a, b in zip(before, (d.q, d.k, d.v, d.pt, d.lens)):
        # compare bytes: the pools hold NaN in slots past each sequence's end
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    check_full(p, o.double().cpu().numpy(), None)


def test_decode_strided_q_and_o():
    """Q and O given through non-packed strides (a slice of a larger buffer)."""
    _say("decode strides")
    p = synth.make_decode(78, 2, 8, 2, 64, [300, 129], 2, kv_dtype=DT_BF16)
    d = Dev(p)
    qbig = torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    qbig[:, :, 4:12] = d.q
    obig = torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    pa.paged_decode(ctx(), qbig[:, :, 4:12], d.k, d.v, d.pt, d.lens, out=obig[:, :, 4:12])
    torch.cuda.synchronize()
    check_full(p, obig[:, :, 4:12].double().cpu().numpy(), None)
    assert torch.all(obig[:, :, :4] == 0) and torch.all(obig[:, :, 12:] == 0)


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    ("d64_g4_sink", dict(B=2, Hq=8, Hkv=2, d=64, S=300, sinks=True)),
    ("d64_g8_cfg4shape", dict(B=1, Hq=64, Hkv=8, d=64, S=260, sinks=True, scale=0.125)),
    ("d128_g4", dict(B=2, Hq=8, Hkv=2, d=128, S=200, sinks=False)),
    ("d64_mha", dict(B=1, Hq=3, Hkv=3, d=64, S=190, sinks=True)),
    ("d128_g3_odd", dict(B=1, Hq=6, Hkv=2, d=128, S=129, sinks=True)),
    ("d64_f16", dict(B=1, Hq=4, Hkv=2, d=64, S=257, sinks=True, dt=DT_F16)),
    ("d128_fp8", dict(B=1, Hq=8, Hkv=2, d=128, S=333, sinks=True, dt=DT_FP8)),
    ("d64_chunked", dict(B=2, Hq=8, Hkv=2, d=64, S=700, q_rows=150, sinks=True)),
    ("d64_tiny", dict(B=2, Hq=4, Hkv=2, d=64, S=5, sinks=True)),
    ("d64_fp32_out", dict(B=1, Hq=4, Hkv=2, d=64, S=150, sinks=True, o=DT_F32)),
    # head_dim 256: the 16-rows-per-wave kernel, 32-key tiles
    ("d256_g2_sink", dict(B=2, Hq=8, Hkv=4, d=256, S=300, sinks=True)),
    ("d256_g4_f16", dict(B=1, Hq=8, Hkv=2, d=256, S=129, sinks=True, dt=DT_F16)),
    ("d256_fp8", dict(B=1, Hq=4, Hkv=2, d=256, S=200, sinks=True, dt=DT_FP8)),
    ("d256_chunked", dict(B=2, Hq=4, Hkv=1, d=256, S=400, q_rows=90, sinks=True)),
    ("d256_tiny", dict(B=2, Hq=4, Hkv=2, d=256, S=5, sinks=True)),
    ("d256_fp32_out", dict(B=1, Hq=4, Hkv=4, d=256, S=140, sinks=False, o=DT_F32)),
    # tile counts around the two-tiles-per-barrier staging: 1, 2, 3 and 4
    # 64-key tiles (d 64/128), 3 and 5 32-key tiles (d 256)
    ("d64_one_tile", dict(B=1, Hq=4, Hkv=2, d=64, S=64, sinks=True)),
    ("d64_two_tiles", dict(B=1, Hq=4, Hkv=2, d=64, S=128, sinks=True)),
    ("d64_three_tiles", dict(B=1, Hq=4, Hkv=2, d=64, S=129, sinks=True)),
    ("d128_four_tiles", dict(B=1, Hq=4, Hkv=2, d=128, S=256, sinks=True)),
    ("d256_three_tiles", dict(B=1, Hq=4, Hkv=2, d=256, S=96, sinks=True)),
    ("d256_five_tiles", dict(B=1, Hq=4, Hkv=2, d=256, S=150, sinks=True)),
]


def _prefill_problem(kw, seed=81):
    return synth.make_prefill(seed, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                              q_rows=kw.get("q_rows"), kv_dtype=kw.get("dt", DT_BF16),
                              sinks=kw.get("sinks", True), softmax_scale=kw.get("scale", 0.0),
                              o_dtype=kw.get("o"))


@pytest.mark.parametrize("name,kw", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_parity(name, kw):
    _say("prefill", name)
    p = _prefill_problem(kw)
    o, l = run(Dev(p))
    check_full(p, o, l, label=name)


def test_prefill_ragged_batch_lengths():
    """Sequences of different lengths with fewer query rows than keys."""
    _say("prefill ragged")
    p = synth.make_prefill(82, 3, 8, 2, 64, 400, q_rows=100, lens=[400, 250, 100], sinks=True)
    o, l = run(Dev(p))
    check_full(p, o, l)


def test_prefill_more_rows_than_keys_gives_empty_rows():
    _say("prefill empty rows")
    p = synth.make_prefill(83, 2, 4, 2, 64, 50, q_rows=80, lens=[50, 10], sinks=True)
    o, l = run(Dev(p))
    check_full(p, o, l)


BS_CASES = [
    ("d128_blk128", dict(S=1000, Hq=8, Hkv=2, d=128, blk=128, mh=1, keep=0.3)),
    ("d64_blk64_perhead", dict(S=700, Hq=8, Hkv=2, d=64, blk=64, mh=2, keep=0.4, sinks=True)),
    ("d64_blk256", dict(S=900, Hq=4, Hkv=2, d=64, blk=256, mh=1, keep=0.5)),
    ("d256_blk64_perhead", dict(S=600, Hq=4, Hkv=2, d=256, blk=64, mh=2, keep=0.4, sinks=True)),
]


@pytest.mark.parametrize("name,kw", BS_CASES, ids=[c[0] for c in BS_CASES])
def test_blocksparse_parity(name, kw):
    _say("blocksparse", name)
    p = synth.make_blocksparse(91, 1, kw["Hq"], kw["Hkv"], kw["d"], kw["S"], mask_block=kw["blk"],
                               mask_heads=kw["mh"], keep_prob=kw["keep"], sinks=kw.get("sinks", False))
    o, l = run(Dev(p))
    check_full(p, o, l, label=name)


def test_blocksparse_random_mask_with_holes():
    """Arbitrary masks, including dropped diagonal blocks (empty rows) and
    entries above the diagonal (ignored)."""
    _say("blocksparse holes")
    p = synth.make_blocksparse(92, 2, 4, 2, 64, 500, mask_block=64, mask_heads=1, sinks=True)
    u = synth.uniform(92, 50, p.mask.numel()).view(p.mask.shape)
    p.mask = (u < 0.5).to(torch.uint8)
    o, l = run(Dev(p))
    check_full(p, o, l)


def test_all_ones_mask_bit_identical_to_dense():
    """Skipping nothing keeps the dense arithmetic bit for bit (Geramy/LSE
    releases, v0.4.14: contributing windows keep arithmetic and ordering)."""
    _say("all-ones mask")
    p = synth.make_blocksparse(93, 2, 8, 2, 128, 600, mask_block=128, sinks=True)
    p.mask = torch.ones_like(p.mask)
    o1, l1 = run(Dev(p))
    p.mask = None
    p.kind = "prefill"
    o0, l0 = run(Dev(p))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_prefill_sink_minus_inf_bit_identical():
    _say("prefill sink -inf")
    p = synth.make_prefill(94, 1, 8, 2, 64, 300, sinks=False)
    o0, l0 = run(Dev(p))
    p.sinks = torch.full((8,), -math.inf, dtype=torch.float32)
    o1, l1 = run(Dev(p))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_prefill_page_permutation_bit_identical():
    _say("prefill permutation")
    p = synth.make_prefill(95, 2, 8, 2, 64, 333, sinks=True)
    o0, l0 = run(Dev(p))
    perm = synth.permutation(95, 9, p.num_pages)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(p.num_pages)
    p.k_pool = p.k_pool[inv].contiguous()
    p.v_pool = p.v_pool[inv].contiguous()
    p.page_table = perm[p.page_table.long()].to(torch.int32)
    o1, l1 = run(Dev(p))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_prefill_row_matches_decode():
    """Prefill row i equals a single-row decode at length i + 1 (rounding aside)."""
    _say("prefill vs decode")
    p = synth.make_prefill(96, 1, 8, 2, 128, 300, sinks=True, o_dtype=DT_F32)
    o, _ = run(Dev(p))
    for i in [0, 63, 64, 200, 299]:
        q1 = synth.make_decode(96, 1, 8, 2, 128, [300], 1, kv_dtype=DT_BF16, o_dtype=DT_F32, sinks=True)
        q1.k_pool, q1.v_pool, q1.page_table, q1.sinks = p.k_pool, p.v_pool, p.page_table, p.sinks
        q1.seq_lens = torch.tensor([i + 1], dtype=torch.int32)
        q1.q = p.q[:, i:i + 1].clone()
        o1, _ = run(Dev(q1))
        assert np.max(np.abs(o1[0, 0] - o[0, i])) <= 1e-2


def test_decode_workspace_reuse():
    """Consecutive calls of different shapes share one workspace (contents
    left by one call never leak into the next)."""
    _say("workspace reuse")
    p1 = synth.make_decode(79, 3, 32, 8, 128, [1500, 700, 2300], 1, kv_dtype=DT_BF16, stride=160)
    p2 = synth.make_decode(80, 3, 32, 8, 128, [2400, 10, 900], 8, kv_dtype=DT_BF16, stride=160)
    d1, d2 = Dev(p1), Dev(p2)
    o1 = torch.empty(d1.q.shape, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty(d2.q.shape, dtype=torch.bfloat16, device="cuda")
    io1, kv1, op1 = pa.make_io(d1.q, o1), pa.make_kv(d1.k, d1.v, d1.pt, d1.lens), pa.make_opts()
    io2, kv2, op2 = pa.make_io(d2.q, o2), pa.make_kv(d2.k, d2.v, d2.pt, d2.lens), pa.make_opts()
    n = max(pa.attn_paged_decode_workspace_bytes(ctx(), io1, kv1, op1),
            pa.attn_paged_decode_workspace_bytes(ctx(), io2, kv2, op2))
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-filled
    for _ in range(2):
        pa.attn_paged_decode(ctx(), io1, kv1, op1, ws)
        pa.attn_paged_decode(ctx(), io2, kv2, op2, ws)
    torch.cuda.synchronize()
    check_full(p1, o1.double().cpu().numpy(), None)
    check_full(p2, o2.double().cpu().numpy(), None)


def test_read_probe_runs_and_keeps_its_sink():
    """The read-only probe is a measurement hook: it must run over every pattern
    and leave the sink alone (the data never XOR to its fixed constant)."""
    _say("read probe")
    buf = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")   # 4 MiB = 1024 4 KiB tiles
    g = torch.Generator().manual_seed(3)
    order = torch.randperm(1024, generator=g).to(torch.int32).cuda()
    order2 = torch.randperm(2048, generator=g).to(torch.int32).cuda()   # 2 KiB tiles
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    pa.attn_debug_read_probe(ctx(), buf, 0, None, sink)
    pa.attn_debug_read_probe(ctx(), buf, 1, order, sink)
    pa.attn_debug_read_probe(ctx(), buf, 2, order2, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


# ---------------------------------------------------------------- ragged rows

@pytest.mark.parametrize("kv_dtype,R,rps,splits", [
    (DT_BF16, 2, [2, 0, 1, 2], 0),          # VALU path (8 rows per KV head)
    (DT_BF16, 2, [1, 2, 2, 0], 5),
    (DT_BF16, 8, [8, 3, 0, 5], 0),          # MFMA path (32 rows per KV head)
    (DT_FP8, 4, [4, 1, 0, 3], 3),
    (DT_F32, 1, [1, 0, 1, 1], 0),
])
def test_decode_ragged_rows(kv_dtype, R, rps, splits):
    _say(f"ragged decode kv={kv_dtype} R={R} rows={rps} splits={splits}")
    p = synth.make_decode(90 + R, 4, 8, 2, 128 if kv_dtype != DT_F32 else 64, [700, 33, 1500, 260], R,
                          kv_dtype=kv_dtype, sinks=True, rows_per_seq=rps)
    o, lse = run(Dev(p), num_splits=splits)
    check_full(p, o, lse)


@pytest.mark.parametrize("masked", [False, True])
def test_prefill_ragged_rows(masked):
    """Chunked prefill with a different chunk length per sequence."""
    _say(f"ragged prefill masked={masked}")
    if masked:
        p = synth.make_blocksparse(93, 3, 8, 2, 64, 640, mask_block=64, mask_heads=2, keep_prob=0.3)
    else:
        p = synth.make_prefill(92, 3, 8, 2, 64, 700, q_rows=300, lens=[400, 350, 700])
    rows = [p.q_rows, 17, 129] if not masked else [640, 0, 200]
    p.rows_per_seq = torch.tensor(rows, dtype=torch.int32)
    o, lse = run(Dev(p))
    check_full(p, o, lse)


@pytest.mark.parametrize("masked", [False, True])
def test_prefill_ragged_rows_d256(masked):
    _say(f"ragged prefill d256 masked={masked}")
    if masked:
        p = synth.make_blocksparse(94, 3, 4, 2, 256, 320, mask_block=64, mask_heads=1, keep_prob=0.4)
        rows = [320, 0, 77]
    else:
        p = synth.make_prefill(95, 3, 4, 2, 256, 350, q_rows=200, lens=[300, 350, 210])
        rows = [200, 33, 129]
    p.rows_per_seq = torch.tensor(rows, dtype=torch.int32)
    o, lse = run(Dev(p))
    check_full(p, o, lse)


@pytest.mark.parametrize("d,Hq,Hkv,S", [(64, 8, 2, 300), (256, 4, 2, 200)])
def test_prefill_replay_deterministic(d, Hq, Hkv, S):
    """Repeated calls give the same bits (a VALU read of an unfinished MFMA
    result would not)."""
    _say(f"prefill replay d={d}")
    p = synth.make_prefill(98, 1, Hq, Hkv, d, S, sinks=True)
    dev = Dev(p)
    o0, l0 = run(dev)
    for _ in range(4):
        o1, l1 = run(dev)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_prefill_d256_row_matches_decode():
    """A prefill row at head_dim 256 equals the single-row decode at its position."""
    _say("prefill d256 row = decode")
    p = synth.make_prefill(96, 1, 4, 2, 256, 200, sinks=True)
    o, _ = run(Dev(p))
    import copy
    i = 137
    q = copy.copy(p)
    q.kind, q.q_rows = "decode", 1
    q.q = p.q[:, i:i + 1].contiguous()
    q.seq_lens = torch.tensor([i + 1], dtype=torch.int32)
    od, _ = run(Dev(q))
    assert np.max(np.abs(o[0, i] - od[0, 0])) <= 2e-2


# ---------------------------------------------------------------- head_dim 256 (decode)

@pytest.mark.parametrize("kv_dtype,R,G", [
    (DT_BF16, 1, 4),      # 4 rows per KV head: the VALU kernel
    (DT_F16, 2, 4),       # 8 rows: the VALU kernel
    (DT_FP8, 4, 4),       # 16 rows: the wide MFMA kernel, one wave of rows
    (DT_BF16, 8, 6),      # 48 rows: three waves
    (DT_F16, 8, 8),       # 64 rows: four waves
    (DT_BF16, 3, 3),      # 9 rows: one partly filled wave
])
def test_decode_head_dim_256(kv_dtype, R, G):
    _say(f"d256 decode kv={kv_dtype} R={R} G={G}")
    p = synth.make_decode(95 + R, 3, 2 * G, 2, 256, [900, 45, 2100], R, kv_dtype=kv_dtype,
                          sinks=True)
    o, lse = run(Dev(p))
    check_full(p, o, lse)
    o2, _ = run(Dev(p), num_splits=7)
    check_full(p, o2, None)


@pytest.mark.parametrize("kv_dtype,R,rps", [(DT_BF16, 4, [4, 1, 0]), (DT_BF8, 8, [8, 3, 6])])
def test_decode_head_dim_256_ragged(kv_dtype, R, rps):
    """Ragged verify rows on the wide kernel (16 and 32 rows per KV head)."""
    _say(f"d256 ragged kv={kv_dtype} R={R} rps={rps}")
    p = synth.make_decode(97, 3, 8, 2, 256, [900, 300, 1700], R, kv_dtype=kv_dtype, sinks=True,
                          rows_per_seq=rps)
    o, lse = run(Dev(p))
    check_full(p, o, lse)
    o2, l2 = run(Dev(p), num_splits=5)
    check_full(p, o2, l2)


def test_gather_head_dim_256():
    p = synth.make_decode(98, 1, 4, 2, 256, [77], 1, kv_dtype=DT_FP8)
    d = Dev(p)
    kv = pa.make_kv(d.k, d.v, d.pt, d.lens, p.k_scale, p.v_scale)
    k_out = torch.full((2, 77, 256), float("nan"), device="cuda")
    v_out = torch.full((2, 77, 256), float("nan"), device="cuda")
    pa.attn_debug_gather_kv(ctx(), kv, 0, 77, k_out, v_out)
    torch.cuda.synchronize()
    for g in range(2):
        k, v = oracle.gather(p, 0, g)
        # the kernels scale in FP32: compare with the FP64 values rounded once to FP32
        assert np.array_equal(k_out[g].double().cpu().numpy(), k.astype(np.float32).astype(np.float64))
        assert np.array_equal(v_out[g].double().cpu().numpy(), v.astype(np.float32).astype(np.float64))
