"""GPU parity at the corners of the definition: sequence lengths beyond the
page table's capacity (clamped to it), block masks smaller than the
sequence's block count (missing entries drop their keys), and calls enqueued
on a stream other than the current one."""
import numpy as np
import pytest
import torch

import paged_gqa_attention_amd as pa
import synth
from synth import DT_BF16, DT_F32, DT_FP8, PAGE

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, ctx, run  # noqa: E402


def _say(*a):
    print(*a, flush=True)


BEYOND = [
    # name, R, d, Hq, Hkv, dtype: VALU (<= 8 rows per KV head), MFMA (16, 32 rows),
    # head_dim 256 VALU and verify kernels, FP32 K/V
    ("valu_r1_bf16", 1, 128, 8, 2, DT_BF16),
    ("valu_r2_f32", 2, 64, 8, 2, DT_F32),
    ("mfma_r4_bf16", 4, 128, 8, 2, DT_BF16),
    ("mfma_r8_fp8", 8, 64, 8, 2, DT_FP8),
    ("valu_r1_d256", 1, 256, 4, 2, DT_BF16),
    ("wide_r8_d256", 8, 256, 8, 2, DT_BF16),
]


@pytest.mark.parametrize("name,R,d,Hq,Hkv,dt", BEYOND, ids=[c[0] for c in BEYOND])
def test_decode_lengths_beyond_capacity(name, R, d, Hq, Hkv, dt):
    """seq_lens above page_table_stride * 16 count as the capacity."""
    _say("decode beyond capacity", name)
    stride = 40
    cap = stride * PAGE
    p = synth.make_decode(241, 3, Hq, Hkv, d, [cap, cap, 300], R, kv_dtype=dt, stride=stride,
                          sinks=True)
    p.seq_lens = torch.tensor([cap + 1, 2 ** 30, 300], dtype=torch.int32)
    o, l = run(Dev(p))
    check_full(p, o, l, label=name)


@pytest.mark.parametrize("d,masked", [(64, False), (128, True), (256, False), (256, True)])
def test_prefill_lengths_beyond_capacity(d, masked):
    _say("prefill beyond capacity", d, masked)
    stride = 20
    cap = stride * PAGE
    if masked:
        p = synth.make_blocksparse(242, 2, 4, 2, d, cap, mask_block=64, keep_prob=0.5, sinks=True)
    else:
        p = synth.make_prefill(242, 2, 4, 2, d, cap, sinks=True)
    assert p.page_table.shape[1] == stride
    p.seq_lens = torch.tensor([cap + 77, 2 ** 30], dtype=torch.int32)
    o, l = run(Dev(p))
    check_full(p, o, l, label=f"d={d} masked={masked}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_blocksparse_mask_smaller_than_the_sequence(d):
    """A mask covering fewer query and key blocks than the sequence has: rows
    of query blocks past its extent keep no key (o = 0, lse = the sink)."""
    _say("blocksparse small mask", d)
    S, blk = 700, 64
    p = synth.make_blocksparse(243, 2, 4, 2, d, S, mask_block=blk, mask_heads=2, keep_prob=0.6,
                               sinks=True)
    p.mask = p.mask[:, :, :7, :4].contiguous()       # 7 of 11 query blocks, 4 of 11 key blocks
    o, l = run(Dev(p))
    check_full(p, o, l, label=f"d={d}")
    assert np.all(o[:, 7 * blk:] == 0)


def test_calls_on_a_side_stream():
    """The convenience calls enqueue on the given stream and allocate their output
    and workspace there; the results equal the current-stream calls'."""
    _say("side stream")
    p = synth.make_decode(244, 4, 16, 4, 128, [3000, 1, 2048, 777], 4, kv_dtype=DT_BF16,
                          sinks=True)
    d = Dev(p)
    o_ref, l_ref = run(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o = pa.paged_decode(ctx(), d.q, d.k, d.v, d.pt, d.lens, sinks=d.sinks, stream=side)
        outs.append(o)
        # work on the current stream that would reuse a freed workspace block
        junk = torch.full((1 << 22,), 7.0, device="cuda")
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.float().cpu(), torch.from_numpy(o_ref).float())
    pf = synth.make_prefill(245, 2, 8, 2, 64, 300, sinks=True)
    dp = Dev(pf)
    o_ref, _ = run(dp)
    side.wait_stream(torch.cuda.current_stream())
    o = pa.prefill(ctx(), dp.q, dp.k, dp.v, dp.pt, dp.lens, sinks=dp.sinks,
                   stream=side.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o.float().cpu(), torch.from_numpy(o_ref).float())
