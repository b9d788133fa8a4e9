"""Shared test plumbing: move a synth.Problem to the GPU, run the library on
it through the C ABI binding, and compare with the FP64 oracle."""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

import oracle
import paged_gqa_attention_amd as pa
import synth

# acceptance bars (max abs error against the oracle)
TOL = {synth.DT_F32: 1e-4, synth.DT_F16: 2e-2, synth.DT_BF16: 2e-2, synth.DT_FP8: 5e-2,
       synth.DT_BF8: 5e-2}
LSE_TOL = {synth.DT_F32: 1e-4, synth.DT_F16: 4e-3, synth.DT_BF16: 4e-3, synth.DT_FP8: 4e-3,
           synth.DT_BF8: 4e-3}

_ctx = None


def ctx():
    global _ctx
    if _ctx is None:
        _ctx = pa.attn_open(0)
    return _ctx


class Dev:
    """Device copies of a problem's tensors."""

    def __init__(self, p: synth.Problem, dev="cuda"):
        self.p = p
        self.k = p.k_pool.to(dev)
        self.v = p.v_pool.to(dev)
        self.pt = p.page_table.to(dev)
        self.lens = p.seq_lens.to(dev)
        self.q = p.q.to(dev)
        self.sinks = p.sinks.to(dev) if p.sinks is not None else None
        self.mask = p.mask.to(dev) if p.mask is not None else None
        self.rows = p.rows_per_seq.to(dev) if p.rows_per_seq is not None else None
        self.k_vs = p.k_vs.to(dev) if p.k_vs is not None else None
        self.v_vs = p.v_vs.to(dev) if p.v_vs is not None else None
        self.o_dtype = synth.TORCH_DTYPE[p.o_dtype]


def run(d: Dev, lse: bool = True, num_splits: int = 0, out_dtype=None):
    """Run the problem's call on the GPU; returns (o float64 numpy, lse numpy or None)."""
    p = d.p
    o = torch.full(d.q.shape, float("nan"), dtype=out_dtype or d.o_dtype, device=d.q.device)
    lse_t = (torch.full((p.batch, p.num_q_heads, p.q_rows), float("nan"), dtype=torch.float32,
                        device=d.q.device) if lse else None)
    if p.kind == "decode":
        pa.paged_decode(ctx(), d.q, d.k, d.v, d.pt, d.lens, k_scale=p.k_scale, v_scale=p.v_scale,
                        softmax_scale=p.softmax_scale, sinks=d.sinks, out=o, lse=lse_t,
                        num_splits=num_splits, rows_per_seq=d.rows, k_vscales=d.k_vs,
                        v_vscales=d.v_vs)
    else:
        pa.prefill(ctx(), d.q, d.k, d.v, d.pt, d.lens, k_scale=p.k_scale, v_scale=p.v_scale,
                   softmax_scale=p.softmax_scale, sinks=d.sinks, out=o, lse=lse_t,
                   block_mask=d.mask, mask_block=p.mask_block, rows_per_seq=d.rows,
                   k_vscales=d.k_vs, v_vscales=d.v_vs)
    torch.cuda.synchronize()
    return (o.to(torch.float64).cpu().numpy(),
            lse_t.to(torch.float64).cpu().numpy() if lse else None)


def max_err(o_gpu, o_ref):
    # rows the oracle marks NaN do not exist (ragged rows): the GPU must have
    # left them untouched (run() pre-fills the outputs with NaN)
    absent = np.isnan(o_ref)
    if absent.any():
        assert np.all(np.isnan(o_gpu[absent])), "a row past its sequence's row count was written"
        o_gpu, o_ref = np.where(absent, 0.0, o_gpu), np.where(absent, 0.0, o_ref)
    diff = np.abs(o_gpu - o_ref)
    if np.isnan(diff).any():
        return math.inf, np.unravel_index(np.argmax(np.isnan(diff)), diff.shape)
    i = np.unravel_index(np.argmax(diff), diff.shape)
    return float(diff[i]), i


def lse_err(l_gpu, l_ref):
    absent = np.isnan(l_ref)
    if absent.any():
        assert np.all(np.isnan(l_gpu[absent])), "an lse past its sequence's row count was written"
        l_gpu, l_ref = np.where(absent, 0.0, l_gpu), np.where(absent, 0.0, l_ref)
    both_inf = np.isneginf(l_gpu) & np.isneginf(l_ref)
    d = np.where(both_inf, 0.0, np.abs(l_gpu - l_ref))
    return float(np.nan_to_num(d, nan=math.inf).max()) if d.size else 0.0


def check_full(p: synth.Problem, o_gpu, l_gpu, tol=None, lse_tol=None, label=""):
    o_ref, l_ref = oracle.attend_full(p)
    tol = tol if tol is not None else TOL[p.kv_dtype]
    err, where = max_err(o_gpu, o_ref)
    assert err <= tol, f"{label} max |o - oracle| = {err} at {where} (tol {tol})"
    if l_gpu is not None:
        lt = lse_tol if lse_tol is not None else LSE_TOL[p.kv_dtype]
        le = lse_err(l_gpu, l_ref)
        assert le <= lt, f"{label} max |lse - oracle| = {le} (tol {lt})"
    return err


def sample_rows(p: synth.Problem, n: int, seed: int = 0) -> np.ndarray:
    """n (b, i, h) triples spread over the output, always including the last
    row of every sequence and the first row."""
    g = np.random.default_rng(seed)
    rows = [(b, p.q_rows - 1, int(g.integers(p.num_q_heads))) for b in range(p.batch)]
    rows.append((0, 0, 0))
    while len(rows) < n:
        rows.append((int(g.integers(p.batch)), int(g.integers(p.q_rows)),
                     int(g.integers(p.num_q_heads))))
    return np.array(rows, dtype=np.int32)


def check_sampled(p: synth.Problem, o_gpu, l_gpu, rows: np.ndarray, label=""):
    o_ref, l_ref, _ = oracle.attend(p, rows)
    got = np.stack([o_gpu[b, i, h] for b, i, h in rows])
    tol = TOL[p.kv_dtype]
    err, where = max_err(got, o_ref)
    assert err <= tol, f"{label} sampled max |o - oracle| = {err} at row {rows[where[0]]} (tol {tol})"
    if l_gpu is not None:
        lg = np.array([l_gpu[b, h, i] for b, i, h in rows])
        le = lse_err(lg, l_ref)
        assert le <= LSE_TOL[p.kv_dtype], f"{label} sampled lse err {le}"
    return err
