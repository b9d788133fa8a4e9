"""Randomised GPU parity: decode, prefill and block-sparse prefill on shapes,
formats, ragged lengths, row counts and forced partition counts drawn from a
fixed seed, each against the FP64 oracle at the usual bars.  The systematic
tests pin each feature; these mix them (every kernel, every K/V format, the
planner's partition sizes and the staging loops' tile counts)."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import synth  # noqa: E402
from synth import DT_BF16, DT_BF8, DT_F16, DT_F32, DT_FP8  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, run  # noqa: E402


def _say(*a):
    print("[random]", *a, flush=True)


def _decode_cases(n=36, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(g.choice([64, 128, 256]))
        kv = int(g.choice([DT_BF16, DT_F16, DT_FP8, DT_BF8] + ([DT_F32] if d != 256 else [])))
        hkv = int(g.choice([1, 2, 4]))
        G = int(g.choice([1, 2, 4, 8]))
        R = int(g.integers(1, 9))
        B = int(g.integers(1, 4))
        lens = [int(x) for x in g.integers(R, 2600, B)]
        rows = [int(x) for x in g.integers(0, R + 1, B)] if g.random() < 0.3 else None
        vs = kv in (DT_FP8, DT_BF8) and g.random() < 0.5
        splits = int(g.choice([0, 0, 1, 3, 7]))
        stride = max((L + 15) // 16 for L in lens) + int(g.integers(0, 40))
        out.append(dict(i=i, d=d, kv=kv, hkv=hkv, G=G, R=R, B=B, lens=lens, rows=rows, vs=vs,
                        splits=splits, stride=stride, sinks=bool(g.random() < 0.6)))
    return out


DECODE = _decode_cases()


@pytest.mark.parametrize("c", DECODE, ids=[f"dec{c['i']}" for c in DECODE])
def test_random_decode(c):
    _say("decode", c)
    p = synth.make_decode(3000 + c["i"], c["B"], c["hkv"] * c["G"], c["hkv"], c["d"], c["lens"],
                          c["R"], kv_dtype=c["kv"], stride=c["stride"], sinks=c["sinks"],
                          rows_per_seq=c["rows"], vscales=c["vs"])
    o, l = run(Dev(p), num_splits=c["splits"])
    check_full(p, o, l, label=f"dec{c['i']}")


def _prefill_cases(n=20, seed=2027):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(g.choice([64, 128, 256]))
        kv = int(g.choice([DT_BF16, DT_F16, DT_FP8, DT_BF8]))
        hkv = int(g.choice([1, 2, 4]))
        G = int(g.choice([1, 2, 3, 4, 8]))
        B = int(g.integers(1, 3))
        S = int(g.integers(1, 700))
        q_rows = int(g.integers(1, S + 1)) if g.random() < 0.3 else None
        vs = kv in (DT_FP8, DT_BF8) and g.random() < 0.4
        sparse = g.random() < 0.35
        out.append(dict(i=i, d=d, kv=kv, hkv=hkv, G=G, B=B, S=S, q_rows=q_rows, vs=vs,
                        sparse=sparse, blk=int(g.choice([64, 128])),
                        keep=float(g.uniform(0.05, 0.6)), sinks=bool(g.random() < 0.6)))
    return out


PREFILL = _prefill_cases()


@pytest.mark.parametrize("c", PREFILL, ids=[f"pre{c['i']}" for c in PREFILL])
def test_random_prefill(c):
    _say("prefill", c)
    if c["sparse"]:
        p = synth.make_blocksparse(4000 + c["i"], c["B"], c["hkv"] * c["G"], c["hkv"], c["d"],
                                   c["S"], mask_block=c["blk"], keep_prob=c["keep"],
                                   sinks=c["sinks"], kv_dtype=c["kv"], vscales=c["vs"])
    else:
        p = synth.make_prefill(4000 + c["i"], c["B"], c["hkv"] * c["G"], c["hkv"], c["d"], c["S"],
                               q_rows=c["q_rows"], kv_dtype=c["kv"], sinks=c["sinks"],
                               vscales=c["vs"])
    o, l = run(Dev(p))
    lse_tol = None
    if c["vs"]:
        import test_gpu_8bit as t8
        lse_tol = t8._prefill_lse_tol(p)
    check_full(p, o, l, lse_tol=lse_tol, label=f"pre{c['i']}")
