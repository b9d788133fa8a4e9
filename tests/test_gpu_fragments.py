"""GPU parity of fragment addressing: the K/V pools split into fragments of
2^s pages placed at shuffled slots of separate arenas and reached through
fragment tables (device addresses).  Every call must give the same bits as
over the contiguous pool (the pages: fragment re-addressing kept outputs
identical), and the oracle's result within the usual bars."""
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

from helpers import Dev, check_full, ctx  # noqa: E402


def _say(*a):
    print("[frag]", *a, flush=True)


class Fragmented:
    """A pool copied into fragments of 2^log2 pages at shuffled arena slots."""

    def __init__(self, pool: torch.Tensor, log2: int, seed: int, spare: int = 3):
        n = pool.shape[0]
        per = 1 << log2
        F = (n + per - 1) // per
        slots = F + spare
        g = torch.Generator().manual_seed(seed)
        perm = torch.randperm(slots, generator=g)[:F]
        shape = (slots, per) + tuple(pool.shape[1:])
        raw = pool.view(torch.uint8) if pool.element_size() == 1 else pool
        arena = torch.full(shape, 0x7F if pool.element_size() == 1 else float("nan"),
                           dtype=raw.dtype, device=pool.device)
        for f in range(F):
            lo, hi = f * per, min(n, f * per + per)
            arena[int(perm[f]), : hi - lo] = raw[lo:hi]
        self.arena = arena.view(pool.dtype) if pool.element_size() == 1 else arena
        self.table = torch.tensor([self.arena[int(perm[f])].data_ptr() for f in range(F)],
                                  dtype=torch.int64, device=pool.device)
        self.view = self.arena[0]          # one fragment: dtype and strides
        self.perm, self.log2, self.num_pages = perm, log2, n

    def read_back(self, like: torch.Tensor) -> torch.Tensor:
        """The pool's pages in page order (to compare after an append)."""
        per = 1 << self.log2
        out = torch.empty_like(like)
        for f in range((self.num_pages + per - 1) // per):
            lo, hi = f * per, min(self.num_pages, f * per + per)
            out[lo:hi] = self.arena[int(self.perm[f]), : hi - lo]
        return out


def _kv(d: Dev, fk=None, fv=None, p=None):
    p = p or d.p
    if fk is None:
        return pa.make_kv(d.k, d.v, d.pt, d.lens, p.k_scale, p.v_scale, d.k_vs, d.v_vs)
    return pa.make_kv(fk.view, fv.view, d.pt, d.lens, p.k_scale, p.v_scale, d.k_vs, d.v_vs,
                      k_fragments=fk.table, v_fragments=fv.table, fragment_pages_log2=fk.log2,
                      num_pages=fk.num_pages)


def _run(d: Dev, kv):
    p = d.p
    o = torch.full(d.q.shape, float("nan"), dtype=d.o_dtype, device="cuda")
    lse = torch.full((p.batch, p.num_q_heads, p.q_rows), float("nan"), dtype=torch.float32,
                     device="cuda")
    io = pa.make_io(d.q, o, lse)
    if p.kind == "decode":
        op = pa.make_opts(p.softmax_scale, d.sinks, rows_per_seq=d.rows)
        ws = pa.decode_workspace(ctx(), io, kv, op, "cuda")
        pa.attn_paged_decode(ctx(), io, kv, op, ws)
    else:
        op = pa.make_opts(p.softmax_scale, d.sinks, d.mask, p.mask_block, rows_per_seq=d.rows)
        (pa.attn_prefill if d.mask is None else pa.attn_prefill_blocksparse)(ctx(), io, kv, op)
    torch.cuda.synchronize()
    return o, lse


def _both(p, log2, seed=5):
    d = Dev(p)
    o0, l0 = _run(d, _kv(d))
    fk, fv = Fragmented(d.k, log2, seed), Fragmented(d.v, log2, seed + 1)
    o1, l1 = _run(d, _kv(d, fk, fv))
    same_o = torch.equal(o0.view(torch.int16) if o0.element_size() == 2 else o0.view(torch.int32),
                         o1.view(torch.int16) if o1.element_size() == 2 else o1.view(torch.int32))
    assert same_o, "fragmented output differs from the contiguous one"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
    check_full(p, o1.double().cpu().numpy(), l1.double().cpu().numpy(), label=f"log2={log2}")


CASES = [
    ("bf16_r1", dict(kind="d", B=3, Hq=32, Hkv=8, d=128, lens=[1000, 37, 2100], R=1, dt=DT_BF16), 3),
    ("bf16_r4_mfma", dict(kind="d", B=2, Hq=32, Hkv=8, d=128, lens=[1000, 2100], R=4, dt=DT_BF16), 2),
    ("f16_r8_d64_single_pages", dict(kind="d", B=2, Hq=8, Hkv=2, d=64, lens=[300, 1029], R=8, dt=DT_F16), 0),
    ("f32_r1", dict(kind="d", B=2, Hq=8, Hkv=2, d=128, lens=[300, 700], R=1, dt=DT_F32), 4),
    ("fp8vs_r4", dict(kind="d", B=2, Hq=32, Hkv=8, d=128, lens=[1500, 777], R=4, dt=DT_FP8, vs=True), 3),
    ("bf8_r1_d256", dict(kind="d", B=2, Hq=8, Hkv=2, d=256, lens=[700, 45], R=1, dt=DT_BF8), 1),
    ("fp8vs_r4_d256_wide", dict(kind="d", B=2, Hq=8, Hkv=2, d=256, lens=[700, 45], R=4, dt=DT_FP8, vs=True), 2),
    ("prefill_bf16_d256", dict(kind="p", B=1, Hq=4, Hkv=2, d=256, S=200, dt=DT_BF16), 3),
    ("prefill_bf16_d64", dict(kind="p", B=2, Hq=8, Hkv=2, d=64, S=300, dt=DT_BF16), 2),
    ("prefill_fp8vs_d128", dict(kind="p", B=1, Hq=8, Hkv=2, d=128, S=333, dt=DT_FP8, vs=True), 5),
    ("sparse_bf8_d128", dict(kind="s", B=1, Hq=8, Hkv=2, d=128, S=1100, dt=DT_BF8), 3),
]


@pytest.mark.parametrize("name,kw,log2", CASES, ids=[c[0] for c in CASES])
def test_fragmented_equals_contiguous(name, kw, log2):
    _say(name, "log2", log2)
    if kw["kind"] == "d":
        p = synth.make_decode(211, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["lens"], kw["R"],
                              kv_dtype=kw["dt"], vscales=kw.get("vs", False), sinks=True,
                              o_dtype=DT_F32 if kw["dt"] == DT_F32 else None,
                              q_dtype=DT_F32 if kw["dt"] == DT_F32 else None)
    elif kw["kind"] == "p":
        p = synth.make_prefill(212, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                               kv_dtype=kw["dt"], vscales=kw.get("vs", False), sinks=True)
    else:
        p = synth.make_blocksparse(213, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                                   keep_prob=0.3, sinks=True, kv_dtype=kw["dt"])
    if kw.get("vs") and kw["kind"] == "p":
        # the prefill LSE bar of per-vector scales comes from the operand rounding
        import test_gpu_8bit as t8
        d = Dev(p)
        o0, l0 = _run(d, _kv(d))
        fk, fv = Fragmented(d.k, log2, 5), Fragmented(d.v, log2, 6)
        o1, l1 = _run(d, _kv(d, fk, fv))
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        check_full(p, o1.double().cpu().numpy(), l1.double().cpu().numpy(),
                   lse_tol=t8._prefill_lse_tol(p), label=name)
        return
    _both(p, log2)


def test_gather_through_fragments():
    _say("gather")
    p = synth.make_decode(214, 2, 4, 2, 64, [70, 33], 1, kv_dtype=DT_FP8, stride=8, vscales=True)
    d = Dev(p)
    fk, fv = Fragmented(d.k, 1, 7), Fragmented(d.v, 1, 8)
    for b in range(2):
        L = int(p.seq_lens[b])
        outs = []
        for kv in (_kv(d), _kv(d, fk, fv)):
            ko = torch.empty((2, L, 64), dtype=torch.float32, device="cuda")
            vo = torch.empty_like(ko)
            pa.attn_debug_gather_kv(ctx(), kv, b, L, ko, vo)
            outs.append((ko, vo))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("kv_dtype,vs", [(DT_BF16, False), (DT_FP8, True)])
def test_append_into_fragments(kv_dtype, vs):
    """The append writes the same bytes into fragments as into the contiguous pool."""
    _say("append", kv_dtype, vs)
    p = synth.make_decode(215, 4, 8, 2, 128, [37, 5, 16, 64], 1, kv_dtype=kv_dtype, stride=5,
                          vscales=vs)
    knew, vnew = synth.append_rows(216, 4, 7, 2, 128, dtype=torch.bfloat16)
    rows = pa.make_rows(knew.cuda(), vnew.cuda())
    d0, d1 = Dev(p), Dev(p)
    pa.attn_kv_append(ctx(), _kv(d0, p=p), rows)
    fk, fv = Fragmented(d1.k, 2, 9), Fragmented(d1.v, 2, 10)
    pa.attn_kv_append(ctx(), _kv(d1, fk, fv, p=p), rows)
    torch.cuda.synchronize()
    kb, vb = fk.read_back(d1.k), fv.read_back(d1.v)
    assert np.array_equal(synth.pool_codes(d0.k), synth.pool_codes(kb))
    assert np.array_equal(synth.pool_codes(d0.v), synth.pool_codes(vb))
    if vs:
        # bit patterns: slots past a sequence's end hold NaN scales
        assert torch.equal(d0.k_vs.view(torch.int32), d1.k_vs.view(torch.int32))
        assert torch.equal(d0.v_vs.view(torch.int32), d1.v_vs.view(torch.int32))
