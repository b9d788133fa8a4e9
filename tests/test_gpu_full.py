"""Full-size parity: the five workloads at their stated sizes, in the launch
configuration the benchmark times (automatic split planning).

Decode workloads (tiny decode, decode/verify at R = 1, 4, 8 with mixed and
uniform lengths, FP8 long decode) are compared with the FP64 oracle on every
output element.  Prefill workloads (all nine (S, B) points of causal prefill
with sinks, and the block-sparse 32K prefill) are compared on the first and
the last row of every (sequence, query head, 128-row query tile): each such
tile is one workgroup's share of the grid, so every workgroup of the
XCD-remapped launch is checked, including its most expensive (last) row.
Every output is also checked finite and, where no sink takes weight, inside
the range of the values (a convex combination: |o| <= max |v|)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, check_sampled, run  # noqa: E402

torch.set_num_threads(min(16, torch.get_num_threads()))


def _say(*a):
    print(*a, flush=True)


def _finite_and_bounded(p, o):
    assert np.isfinite(o).all()
    vmax = float(p.v_pool.float().nan_to_num(0).abs().max()) * p.v_scale
    assert np.abs(o).max() <= vmax * (1 + 1e-2)


def _tile_rows(p, tile=128):
    """(b, i, h) of the first and last row of every (sequence, head, query tile)."""
    rows = []
    for b in range(p.batch):
        for t0 in range(0, p.q_rows, tile):
            t1 = min(p.q_rows, t0 + tile) - 1
            for h in range(p.num_q_heads):
                rows.append((b, t0, h))
                rows.append((b, t1, h))
    return np.array(rows, dtype=np.int32)


def test_config1_tiny_decode():
    _say("config1")
    p = synth.config1()
    o, l = run(Dev(p))
    check_full(p, o, l, label="cfg1")


@pytest.mark.parametrize("R", [1, 4, 8])
def test_config2_decode_verify_mixed_lengths(R):
    _say("config2 mixed lengths R", R)
    p = synth.config2(q_rows=R, device="cuda")
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_full(p, o, l, label=f"cfg2 R={R}")


@pytest.mark.parametrize("R", [1, 4, 8])
def test_config2_uniform_16k(R):
    _say("config2 16K R", R)
    p = synth.config2(q_rows=R, lens=[16384] * 16, device="cuda")
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_full(p, o, l, label=f"cfg2 16K R={R}")


def test_config3_fp8_long_decode():
    _say("config3")
    p = synth.config3(device="cuda")
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_full(p, o, l, label="cfg3")


@pytest.mark.parametrize("S", [1024, 4096, 8192])
@pytest.mark.parametrize("B", [1, 4, 16])
def test_config4_prefill_sinks(S, B):
    _say("config4", S, B)
    p = synth.config4(seq_len=S, batch=B, device="cuda")
    o, l = run(Dev(p))
    assert np.isfinite(o).all()
    rows = _tile_rows(p)
    _say("  rows", len(rows))
    check_sampled(p, o, l, rows, label=f"cfg4 S={S} B={B}")


def test_config5_blocksparse():
    _say("config5")
    p = synth.config5(device="cuda")
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    # plus rows whose query block keeps only block 0 and the diagonal
    m = p.mask[0, 0].cpu()
    lone = [qb for qb in range(1, m.shape[0]) if int(m[qb, :qb + 1].sum()) <= 2][:4]
    extra = [(0, 128 * qb + 5, 3) for qb in lone]
    rows = np.concatenate([_tile_rows(p), np.array(extra, dtype=np.int32).reshape(-1, 3)])
    _say("  rows", len(rows))
    check_sampled(p, o, l, rows, label="cfg5")
