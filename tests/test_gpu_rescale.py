"""GPU parity where the running maximum must move during a row: scores that
rise along the sequence by more than the exponentials' bound per tile (the
reference maximum is refreshed on every tile), one jump in the middle, and a
first tile far above the rest (later exponentials underflow against it).  The
inputs are the seeded synthetic problems with a ramp added along one fixed
direction of K and Q; the oracle sees the same stored codes."""
import pytest
import torch

import synth
from synth import DT_BF16, DT_F16

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, run  # noqa: E402


def _shape(p, amp_of):
    """K[token] += amp_of(token) * u and Q[row] += 4 u for a fixed unit vector u,
    so every score gains 4 * amp_of(key)."""
    d = p.head_dim
    g = torch.Generator().manual_seed(5)
    u = torch.randn(d, generator=g, dtype=torch.float64)
    u /= u.norm()
    k = p.k_pool.to(torch.float64)
    for b in range(p.batch):
        for j in range(int(p.seq_lens[b])):
            k[int(p.page_table[b, j // 16]), :, j % 16, :] += amp_of(j) * u
    p.k_pool = k.to(p.k_pool.dtype)
    p.q = (p.q.to(torch.float64) + 4.0 * u).to(p.q.dtype)
    return p


def _ramp(slope):
    return lambda j: slope * j


def _jump(at, by):
    return lambda j: by if j >= at else 0.0


def _first_high(by):
    return lambda j: by if j < 40 else 0.0


CASES = [
    # (name, kind, problem kwargs, amplitude profile)
    ("prefill_d64_bf16_ramp", "prefill", dict(B=2, Hq=8, Hkv=2, d=64, S=700, dt=DT_BF16), _ramp(0.5)),
    ("prefill_d64_f16_ramp", "prefill", dict(B=1, Hq=8, Hkv=2, d=64, S=520, dt=DT_F16), _ramp(0.5)),
    ("prefill_d64_bf16_chunk_ramp", "prefill", dict(B=2, Hq=8, Hkv=2, d=64, S=700, q_rows=150, dt=DT_BF16), _ramp(0.5)),
    ("prefill_d64_bf16_jump", "prefill", dict(B=1, Hq=8, Hkv=2, d=64, S=600, dt=DT_BF16), _jump(300, 50.0)),
    ("prefill_d64_bf16_first_high", "prefill", dict(B=1, Hq=8, Hkv=2, d=64, S=600, dt=DT_BF16), _first_high(60.0)),
    ("prefill_d128_bf16_ramp", "prefill", dict(B=1, Hq=8, Hkv=2, d=128, S=520, dt=DT_BF16), _ramp(0.5)),
    ("prefill_d64_mha_ramp", "prefill", dict(B=1, Hq=3, Hkv=3, d=64, S=400, dt=DT_BF16), _ramp(0.5)),
    ("blocksparse_d64_bf16_ramp", "blocksparse", dict(B=1, Hq=8, Hkv=2, d=64, S=1024, dt=DT_BF16), _ramp(0.25)),
    ("decode_r1_bf16_ramp", "decode", dict(B=2, Hq=8, Hkv=2, d=128, S=3000, R=1, dt=DT_BF16), _ramp(0.2)),
    ("decode_r4_bf16_ramp", "decode", dict(B=2, Hq=8, Hkv=2, d=128, S=3000, R=4, dt=DT_BF16), _ramp(0.2)),
]


def _problem(kind, kw):
    if kind == "prefill":
        return synth.make_prefill(71, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                                  q_rows=kw.get("q_rows"), kv_dtype=kw["dt"], sinks=True)
    if kind == "blocksparse":
        return synth.make_blocksparse(72, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], kw["S"],
                                      mask_block=128, keep_prob=0.5, sinks=True)
    return synth.make_decode(73, kw["B"], kw["Hq"], kw["Hkv"], kw["d"], [kw["S"]] * kw["B"],
                             q_rows=kw["R"], kv_dtype=kw["dt"], sinks=True)


@pytest.mark.parametrize("name,kind,kw,amp", CASES, ids=[c[0] for c in CASES])
def test_running_maximum_moves(name, kind, kw, amp):
    print("rescale", name, flush=True)
    p = _shape(_problem(kind, kw), amp)
    o, lse = run(Dev(p))
    check_full(p, o, lse, label=name)
