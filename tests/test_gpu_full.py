"""Full-size parity: the five workloads at their stated sizes, in the launch
configuration the benchmark times (automatic split planning), checked on
sampled output rows that the oracle computes one by one, plus properties
that hold at any size (finite outputs, sink-free rows are convex
combinations of values: |o| <= max |v|)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_sampled, run, sample_rows  # noqa: E402

torch.set_num_threads(min(16, torch.get_num_threads()))


def _say(*a):
    print(*a, flush=True)


def _finite_and_bounded(p, o):
    assert np.isfinite(o).all()
    vmax = float(p.v_pool.float().nan_to_num(0).abs().max()) * p.v_scale
    assert np.abs(o).max() <= vmax * (1 + 1e-2)


@pytest.mark.parametrize("R", [1, 4, 8])
def test_config2_decode_verify(R):
    _say("config2 R", R)
    p = synth.config2(q_rows=R)
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_sampled(p, o, l, sample_rows(p, 64, seed=R), label=f"cfg2 R={R}")


def test_config2_headline_16k():
    _say("config2 16K")
    p = synth.config2(q_rows=1, lens=[16384] * 16)
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_sampled(p, o, l, sample_rows(p, 64, seed=7), label="cfg2 16K")


def test_config3_fp8_long_decode():
    _say("config3")
    p = synth.config3()
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    check_sampled(p, o, l, sample_rows(p, 48, seed=3), label="cfg3")


@pytest.mark.parametrize("S,B", [(1024, 16), (4096, 4), (8192, 16)])
def test_config4_prefill_sinks(S, B):
    _say("config4", S, B)
    p = synth.config4(seq_len=S, batch=B)
    o, l = run(Dev(p))
    assert np.isfinite(o).all()
    check_sampled(p, o, l, sample_rows(p, 64, seed=S + B), label=f"cfg4 S={S} B={B}")


def test_config5_blocksparse():
    _say("config5")
    p = synth.config5()
    o, l = run(Dev(p))
    _finite_and_bounded(p, o)
    rows = sample_rows(p, 64, seed=5)
    # include rows whose query block keeps only block 0 and the diagonal
    rows = np.concatenate([rows, np.array([[0, 128 * 7 + 5, 3], [0, 32767, 31]], dtype=np.int32)])
    check_sampled(p, o, l, rows, label="cfg5")
