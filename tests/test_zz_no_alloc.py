"""attn_paged_decode_noalloc (device-resident scratch, no allocation) against
attn_paged_decode with a caller workspace: bit-identical outputs and LSE on
two calls in a row, the second with a smaller input, and both within the
oracle's bar; a request beyond the scratch is rejected before any launch."""
import numpy as np
import pytest
import torch

import paged_gqa_attention_amd as pa
import synth
from synth import DT_BF16, DT_FP8

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from helpers import Dev, check_full, ctx  # noqa: E402


def _say(*a):
    print(*a, flush=True)


def _args(d: Dev, lse=True):
    p = d.p
    o = torch.full(d.q.shape, float("nan"), dtype=d.o_dtype, device="cuda")
    l = (torch.full((p.batch, p.num_q_heads, p.q_rows), float("nan"), dtype=torch.float32,
                    device="cuda") if lse else None)
    io = pa.make_io(d.q, o, l)
    kv = pa.make_kv(d.k, d.v, d.pt, d.lens, p.k_scale, p.v_scale, d.k_vs, d.v_vs)
    op = pa.make_opts(p.softmax_scale, d.sinks, None, 128, 0, d.rows)
    return io, kv, op, o, l


def _with_workspace(d: Dev):
    io, kv, op, o, l = _args(d)
    ws = pa.decode_workspace(ctx(), io, kv, op, "cuda")
    pa.attn_paged_decode(ctx(), io, kv, op, ws)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def _noalloc(d: Dev):
    io, kv, op, o, l = _args(d)
    pa.attn_paged_decode_noalloc(ctx(), io, kv, op)
    return io, o, l


def test_noalloc_matches_workspace_call_twice_in_a_row():
    # first a larger call (multi-row verify on the MFMA kernel, 16 x 4,096 tokens),
    # then a smaller one (single-row decode on the VALU kernel, FP8 K/V)
    big = synth.make_decode(261, 16, 32, 8, 128, [4096] * 15 + [999], 4, kv_dtype=DT_BF16,
                            sinks=True)
    small = synth.make_decode(262, 3, 8, 2, 64, [700, 33, 1], 1, kv_dtype=DT_FP8, sinks=True)
    dev = [Dev(big), Dev(small)]
    refs = [_with_workspace(d) for d in dev]
    outs = []
    for d in dev:                       # back to back on one stream
        _say("noalloc call", d.p.batch, d.p.q_rows)
        outs.append(_noalloc(d))
    torch.cuda.synchronize()
    for d, (o_ref, l_ref), (_, o, l) in zip(dev, refs, outs):
        o_na, l_na = o.double().cpu().numpy(), l.double().cpu().numpy()
        assert np.array_equal(o_na, o_ref, equal_nan=True)
        assert np.array_equal(l_na, l_ref, equal_nan=True)
        check_full(d.p, o_na, l_na, label=f"noalloc B={d.p.batch}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    p = synth.make_decode(263, 16, 32, 8, 128, [1024] * 16, 1, kv_dtype=DT_BF16, stride=1024)
    d = Dev(p)
    io, kv, op, o, l = _args(d)
    op.num_splits = 128
    _, _, need = pa.attn_paged_decode_plan(ctx(), io, kv, op)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pa.AttnError) as e:
        pa.attn_paged_decode_noalloc(ctx(), io, kv, op)
    assert e.value.status == pa.ATTN_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()         # nothing was launched
