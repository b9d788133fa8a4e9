"""GPU parity of the 8-bit cache formats beyond per-tensor e4m3fn: OCP e5m2
(BF8) storage and per-vector FP32 scales (one per K or V vector of a token and
head) for both 8-bit formats.  Decode (VALU and MFMA kernels), verify, ragged
rows, prefill, block-sparse prefill and the debug gather are compared with the
FP64 oracle; the K/V append with per-vector scales is compared byte for byte
(codes and scales) with the oracle's append reference."""
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

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, ctx, run  # noqa: E402


def _say(*a):
    print("[8bit]", *a, flush=True)


# ------------------------------------------------------------------ gather / codecs

def test_bf8_every_code_decodes_exactly():
    """All 256 e5m2 codes through the kernels' FP32 and 16-bit conversions."""
    _say("bf8 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    k = codes.view(1, 1, 16, 16).repeat(1, 1, 1, 4).contiguous().view(torch.float8_e5m2)
    v = k.transpose(2, 3).contiguous()
    pt = torch.zeros((1, 1), dtype=torch.int32)
    lens = torch.tensor([16], dtype=torch.int32)
    kv = pa.make_kv(k.cuda(), v.cuda(), pt.cuda(), lens.cuda())
    ko = torch.empty((1, 16, 64), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    pa.attn_debug_gather_kv(ctx(), kv, 0, 16, ko, vo)
    torch.cuda.synchronize()
    ref = oracle.decode_codes(DT_BF8, k.view(torch.uint8).numpy().reshape(-1)).reshape(16, 64)
    nan = np.isnan(ref)
    # the V tile is the K tile transposed, so both gathers return the same [token][d] array
    for got in (ko[0].double().cpu().numpy(), vo[0].double().cpu().numpy()):
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dtype,vscales", [(DT_BF8, False), (DT_FP8, True), (DT_BF8, True)])
def test_gather_scaled_bit_exact(dtype, vscales):
    """(code * per-vector scale) * per-tensor scale in FP32, as the header defines it."""
    _say("gather", dtype, vscales)
    p = synth.make_decode(161, 2, 4, 2, 64, [70, 33], 1, kv_dtype=dtype, stride=8, extra_pages=3,
                          vscales=vscales)
    d = Dev(p)
    for b in range(2):
        L = int(p.seq_lens[b])
        ko = torch.empty((2, L, 64), dtype=torch.float32, device="cuda")
        vo = torch.empty_like(ko)
        kv = pa.make_kv(d.k, d.v, d.pt, d.lens, p.k_scale, p.v_scale, d.k_vs, d.v_vs)
        pa.attn_debug_gather_kv(ctx(), kv, b, L, ko, vo)
        torch.cuda.synchronize()
        kc, vc = synth.logical_kv_codes(p, b)
        kval = oracle.decode_codes(dtype, kc.view(torch.uint8).numpy().reshape(-1)).reshape(2, L, 64)
        vval = oracle.decode_codes(dtype, vc.view(torch.uint8).numpy().reshape(-1)).reshape(2, L, 64)
        kval, vval = kval.astype(np.float32), vval.astype(np.float32)       # exact
        if vscales:
            ks, vs = (t.numpy()[..., None] for t in synth.logical_vscales(p, b))
            kval, vval = (kval * ks).astype(np.float32), (vval * vs).astype(np.float32)
        kref = (kval * np.float32(p.k_scale)).astype(np.float32)
        vref = (vval * np.float32(p.v_scale)).astype(np.float32)
        assert np.array_equal(ko.cpu().numpy(), kref)
        assert np.array_equal(vo.cpu().numpy(), vref)


# ------------------------------------------------------------------ decode / verify

DECODE_CASES = [
    # per-tensor e5m2
    ("bf8_r1", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=1, dt=DT_BF8, sinks=True)),
    ("bf8_r4_mfma", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=4, dt=DT_BF8)),
    ("bf8_r8_d64_f16q", dict(B=2, Hq=16, Hkv=2, d=64, lens=[600, 90], R=8, dt=DT_BF8, q=DT_F16)),
    # per-vector scales
    ("fp8vs_r1", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=1, dt=DT_FP8, vs=True,
                      sinks=True)),
    ("fp8vs_r4_mfma", dict(B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=4, dt=DT_FP8, vs=True)),
    ("bf8vs_r1_d64", dict(B=3, Hq=8, Hkv=2, d=64, lens=[300, 1029, 17], R=1, dt=DT_BF8, vs=True)),
    ("bf8vs_r8_d64_f16q", dict(B=2, Hq=16, Hkv=2, d=64, lens=[600, 90], R=8, dt=DT_BF8, vs=True,
                               q=DT_F16, sinks=True)),
    ("fp8vs_r2_valu8", dict(B=2, Hq=8, Hkv=2, d=128, lens=[515, 1700], R=2, dt=DT_FP8, vs=True)),
    ("fp8vs_r1_d256", dict(B=2, Hq=8, Hkv=2, d=256, lens=[700, 45], R=1, dt=DT_FP8, vs=True)),
    ("bf8vs_r4_d256", dict(B=1, Hq=8, Hkv=4, d=256, lens=[333], R=4, dt=DT_BF8, vs=True)),
    ("bf8vs_r8_64rows", dict(B=1, Hq=16, Hkv=2, d=128, lens=[1100], R=8, dt=DT_BF8, vs=True)),
    ("fp8vs_empty_short", dict(B=3, Hq=8, Hkv=2, d=128, lens=[0, 3, 50], R=4, dt=DT_FP8, vs=True,
                               sinks=True)),
]


def _decode_problem(kw, seed=171):
    return synth.make_decode(seed, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["lens"], kw["R"],
                             kv_dtype=kw["dt"], q_dtype=kw.get("q"), sinks=kw.get("sinks", False),
                             vscales=kw.get("vs", False), rows_per_seq=kw.get("rps"))


@pytest.mark.parametrize("name,kw", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(name, kw):
    _say("decode", name)
    p = _decode_problem(kw)
    o, l = run(Dev(p))
    check_full(p, o, l, label=name)


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_decode_forced_splits_per_vector(splits):
    """Partition boundaries inside pages: the scales follow their tokens."""
    _say("decode splits", splits)
    p = synth.make_decode(172, 2, 16, 4, 128, [2000, 901], 4, kv_dtype=DT_FP8, vscales=True)
    o, l = run(Dev(p), num_splits=splits)
    check_full(p, o, l, label=f"splits={splits}")


@pytest.mark.parametrize("dt,R,rps", [(DT_FP8, 4, [4, 1, 0, 3]), (DT_BF8, 8, [8, 2, 5])])
def test_decode_ragged_rows_per_vector(dt, R, rps):
    _say("decode ragged", dt, R, rps)
    B = len(rps)
    p = synth.make_decode(173, B, 16, 4, 128, [900, 400, 1300, 77][:B], R, kv_dtype=dt,
                          vscales=True, rows_per_seq=rps)
    o, l = run(Dev(p))
    check_full(p, o, l, label=f"ragged {dt} {rps}")


def test_uniform_vector_scales_equal_per_tensor_scale():
    """Every per-vector scale = c must give the per-tensor result with scale c, up to
    where the FP32 roundings fall (per token instead of once per call) and the
    single-row path's 16-bit softmax weights.  Per-tensor scales: each weight is
    rounded to f16 (relative error <= 2^-11) and the row sum uses the rounded
    weights, so the output moves by at most 2^-11 * max|v - o| <= 2^-10 * max|v|.
    Per-vector scales: each weight times its V scale is rounded to bf16 (<= 2^-9)
    under an unrounded row sum, so the output moves by at most 2^-9 * max|v|."""
    _say("uniform scales")
    p = synth.make_decode(174, 2, 8, 2, 128, [700, 300], 1, kv_dtype=DT_BF8)
    d = Dev(p)
    c = 0.0375
    ks = torch.full((p.num_pages, 2, 16), c, dtype=torch.float32, device="cuda")
    o1 = pa.paged_decode(ctx(), d.q, d.k, d.v, d.pt, d.lens, k_scale=c, v_scale=c,
                         out_dtype=torch.float32)
    o2 = pa.paged_decode(ctx(), d.q, d.k, d.v, d.pt, d.lens, k_vscales=ks, v_vscales=ks.clone(),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = (o1 - o2).abs().max().item()
    vmax = torch.nan_to_num(p.v_pool.float(), nan=0.0, posinf=0.0, neginf=0.0).abs().max().item() * c
    assert err <= (2.0 ** -10 + 2.0 ** -9) * vmax + 1e-4, (err, vmax)


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    ("bf8_d64", dict(B=2, Hq=8, Hkv=2, d=64, S=300, dt=DT_BF8)),
    ("bf8_d128", dict(B=1, Hq=8, Hkv=2, d=128, S=333, dt=DT_BF8)),
    ("fp8vs_d64_g8", dict(B=1, Hq=64, Hkv=8, d=64, S=260, dt=DT_FP8, vs=True, scale=0.125)),
    ("fp8vs_d128", dict(B=2, Hq=8, Hkv=2, d=128, S=200, dt=DT_FP8, vs=True)),
    ("bf8vs_d64_g3", dict(B=1, Hq=6, Hkv=2, d=64, S=129, dt=DT_BF8, vs=True)),
    ("bf8vs_d128_chunked", dict(B=2, Hq=8, Hkv=2, d=128, S=700, q_rows=150, dt=DT_BF8, vs=True)),
    ("fp8vs_tiny", dict(B=2, Hq=4, Hkv=2, d=64, S=5, dt=DT_FP8, vs=True)),
    ("bf8vs_d256", dict(B=1, Hq=8, Hkv=2, d=256, S=250, dt=DT_BF8, vs=True)),
    ("bf8_d256", dict(B=1, Hq=4, Hkv=2, d=256, S=170, dt=DT_BF8)),
]


def _prefill_lse_tol(p):
    """LSE bound of the prefill MFMA path with per-vector scales.  Staging rounds
    each dequantised K value (code x scale) once to the bf16 operand (relative
    error <= 2^-9), so a score moves by at most scale * 2^-9 * sum_c |q_c k_c|;
    the LSE moves by at most the largest such shift, plus 2^-9 for the row sum
    of the bf16-rounded weights."""
    if p.k_vs is None:
        return None
    worst = 0.0
    G = p.num_q_heads // p.num_kv_heads
    for b in range(p.batch):
        kc, _ = synth.logical_kv_codes(p, b)
        ks, _ = synth.logical_vscales(p, b)
        kval = oracle.decode_codes(p.kv_dtype, kc.view(torch.uint8).numpy().reshape(-1))
        kval = np.abs(kval.reshape(kc.shape) * ks.numpy()[..., None])          # [Hkv][L][d]
        q = np.abs(p.q[b].double().numpy())                                    # [rows][Hq][d]
        for h in range(p.num_q_heads):
            worst = max(worst, float((q[:, h, :] @ kval[h // G].T).max()))
    return 2.0 ** -9 + p.scale * 2.0 ** -9 * worst + 1e-3


@pytest.mark.parametrize("name,kw", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_parity(name, kw):
    _say("prefill", name)
    p = synth.make_prefill(181, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                           q_rows=kw.get("q_rows"), kv_dtype=kw["dt"], sinks=True,
                           softmax_scale=kw.get("scale", 0.0), vscales=kw.get("vs", False))
    o, l = run(Dev(p))
    check_full(p, o, l, lse_tol=_prefill_lse_tol(p), label=name)


def test_prefill_per_vector_f16_queries():
    _say("prefill f16 q")
    p = synth.make_prefill(182, 1, 8, 2, 64, 300, kv_dtype=DT_BF8, sinks=True, vscales=True)
    p.q = p.q.to(torch.float16)
    p.q_dtype = DT_F16
    p.o_dtype = DT_F16
    o, l = run(Dev(p))
    check_full(p, o, l, lse_tol=_prefill_lse_tol(p), label="prefill f16 q")


@pytest.mark.parametrize("dt", [DT_FP8, DT_BF8])
def test_blocksparse_per_vector(dt):
    _say("blocksparse", dt)
    p = synth.make_blocksparse(183, 1, 8, 2, 128, 1100, mask_block=128, keep_prob=0.3,
                               sinks=True, kv_dtype=dt, vscales=True)
    o, l = run(Dev(p))
    check_full(p, o, l, lse_tol=_prefill_lse_tol(p), label=f"blocksparse {dt}")


# ------------------------------------------------------------------ append

SRC = {DT_F32: torch.float32, DT_F16: torch.float16, DT_BF16: torch.bfloat16}


def _specials(x: torch.Tensor, seed: int):
    """A zero vector, vectors holding NaN / +-inf, huge and tiny magnitudes."""
    g = torch.Generator().manual_seed(seed)
    B, n, H, d = x.shape
    x[0, 0, 0] = 0.0                                            # all zero: scale 1
    x[0, 0, 1, 3] = float("nan")
    x[0, 0, 1, 5] = float("inf")
    if n > 1:
        x[0, 1, 0, :] = 1e-30 if x.dtype == torch.float32 else 1e-6
        x[0, 1, 1, 7] = -float("inf")
    if n > 2:
        x[0, 2, 0] *= 1e4 if x.dtype != torch.float16 else 50.0
    idx = torch.randint(0, x.numel(), (16,), generator=g)
    x.view(-1)[idx] = (x.view(-1)[idx] * 3).to(x.dtype)


def _append_vs(seed, kv_dtype, src_dtype, d, lens, n_new, stride, specials=False, hkv=2):
    p = synth.make_decode(seed, len(lens), 4 * hkv, hkv, d, lens, 1, kv_dtype=kv_dtype,
                          stride=stride, vscales=True)
    knew, vnew = synth.append_rows(seed + 1, len(lens), n_new, hkv, d, dtype=SRC[src_dtype])
    if specials:
        _specials(knew, seed)
        _specials(vnew, seed + 7)
    k0, v0 = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    kexp, vexp, ksexp, vsexp = oracle.kv_append(
        kv_dtype, k0, v0, p.page_table.numpy(), p.seq_lens.numpy(), knew.float().numpy(),
        vnew.float().numpy(), k_vs=p.k_vs.numpy(), v_vs=p.v_vs.numpy())
    dev = Dev(p)
    _say(f"append seed={seed} kv={kv_dtype} src={src_dtype} d={d} lens={lens} n_new={n_new}")
    kv = pa.make_kv(dev.k, dev.v, dev.pt, dev.lens, 1.0, 1.0, dev.k_vs, dev.v_vs)
    pa.attn_kv_append(ctx(), kv, pa.make_rows(knew.cuda(), vnew.cuda()))
    torch.cuda.synchronize()
    got = (synth.pool_codes(dev.k), synth.pool_codes(dev.v), dev.k_vs.cpu().numpy(),
           dev.v_vs.cpu().numpy())
    return p, dev, got, (kexp, vexp, ksexp, vsexp)


def _same(a, b):
    return np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                          b.view(np.uint32) if b.dtype == np.float32 else b)


@pytest.mark.parametrize("kv_dtype", [DT_FP8, DT_BF8])
@pytest.mark.parametrize("src_dtype", [DT_F32, DT_F16, DT_BF16])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_append_per_vector_bit_exact(kv_dtype, src_dtype, d):
    p, dev, got, exp = _append_vs(191 + d, kv_dtype, src_dtype, d, [37, 5, 16, 64], 7, 5,
                                  specials=True)
    for g_, e_, what in zip(got, exp, ("K codes", "V codes", "K scales", "V scales")):
        assert _same(g_, e_), f"{what} differ"


@pytest.mark.parametrize("src_dtype", [DT_F32, DT_BF16])
def test_append_bf8_per_tensor_bit_exact(src_dtype):
    seed, lens, n_new = 195, [37, 5, 16, 64], 7
    p = synth.make_decode(seed, 4, 8, 2, 128, lens, 1, kv_dtype=DT_BF8, stride=5)
    knew, vnew = synth.append_rows(seed + 1, 4, n_new, 2, 128, dtype=SRC[src_dtype])
    _specials(knew, seed)
    knew[1, 0, 0, :4] = torch.tensor([6e4, -1e5, 57344.0, 61440.0]).to(knew.dtype)   # saturate
    k0, v0 = synth.pool_codes(p.k_pool), synth.pool_codes(p.v_pool)
    kexp, vexp = oracle.kv_append(DT_BF8, k0, v0, p.page_table.numpy(), p.seq_lens.numpy(),
                                  knew.float().numpy(), vnew.float().numpy(), p.k_scale, p.v_scale)
    dev = Dev(p)
    kv = pa.make_kv(dev.k, dev.v, dev.pt, dev.lens, p.k_scale, p.v_scale)
    pa.attn_kv_append(ctx(), kv, pa.make_rows(knew.cuda(), vnew.cuda()))
    torch.cuda.synchronize()
    assert np.array_equal(synth.pool_codes(dev.k), kexp)
    assert np.array_equal(synth.pool_codes(dev.v), vexp)


@pytest.mark.parametrize("kv_dtype", [DT_FP8, DT_BF8])
def test_attention_over_per_vector_appended_cache(kv_dtype):
    """Append the last 40 rows, then decode (R=4) and prefill over the result."""
    p, dev, got, exp = _append_vs(197, kv_dtype, DT_BF16, 128, [300, 517], 40, 40)
    assert all(_same(g_, e_) for g_, e_ in zip(got, exp))
    p2 = synth.with_pool_codes(p, exp[0], exp[1])
    p2.k_vs, p2.v_vs = torch.from_numpy(exp[2]), torch.from_numpy(exp[3])
    p2.q_rows = 4
    p2.q = synth.quantize(synth.normal(198, 3, (2, 4, 8, 128)), DT_BF16)
    o, l = run(Dev(p2))
    check_full(p2, o, l, label="decode over appended")
