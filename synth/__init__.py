"""Seeded synthetic inputs for paged grouped-query attention.

This module only *produces inputs*: random numbers, their rounding to the
storage dtype, the shuffled page pool, page tables, sequence lengths, sink
logits and block masks.  It contains none of the attention arithmetic, so
both the FP64 oracle and the HIP path can consume what it makes without
sharing any of the computation they are compared on.

Random numbers come from a counter-based generator: element ``i`` of stream
``s`` under seed ``k`` is ``mix64(base(k, s) + (i + 1) * 0x9E3779B97F4A7C15)``
where ``mix64`` is the SplitMix64 finaliser (Steele, Lea, Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014).  Uniforms use the
top 53 bits; normals use the Box-Muller transform on consecutive uniform
pairs.  Everything is computed with torch integer/float64 ops, so the bits
are identical on any host and can be produced on the CPU or on a GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
C1 = 0xBF58476D1CE4E5B9
C2 = 0x94D049BB133111EB

PAGE = 16  # tokens per KV page

DT_F32, DT_F16, DT_BF16, DT_FP8, DT_BF8 = 0, 1, 2, 3, 4
TORCH_DTYPE = {
    DT_F32: torch.float32,
    DT_F16: torch.float16,
    DT_BF16: torch.bfloat16,
    DT_FP8: torch.float8_e4m3fn,
    DT_BF8: torch.float8_e5m2,
}
DT_NAMES = {"f32": DT_F32, "f16": DT_F16, "bf16": DT_BF16, "fp8": DT_FP8, "bf8": DT_BF8}
EIGHT_BIT = (DT_FP8, DT_BF8)


def _s64(u: int) -> int:
    """Reinterpret an unsigned 64-bit integer as a signed one (torch int64)."""
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * C1) & MASK64
    z = ((z ^ (z >> 27)) * C2) & MASK64
    return z ^ (z >> 31)


def _lsr(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 tensors holding unsigned 64-bit patterns."""
    return torch.bitwise_and(torch.bitwise_right_shift(x, s), (1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = torch.bitwise_xor(z, _lsr(z, 30)) * _s64(C1)
    z = torch.bitwise_xor(z, _lsr(z, 27)) * _s64(C2)
    return torch.bitwise_xor(z, _lsr(z, 31))


def stream_base(seed: int, stream: int) -> int:
    return _mix64_int(_mix64_int(seed) ^ ((stream * 0xD1B54A32D192ED03) & MASK64))


def raw64(seed: int, stream: int, start: int, n: int, device="cpu") -> torch.Tensor:
    """n raw 64-bit outputs (as int64 bit patterns) of stream ``stream``."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = _s64(stream_base(seed, stream)) + idx * _s64(GOLDEN)
    return _mix64(z)


def uniform(seed: int, stream: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n float64 uniforms in (0, 1)."""
    r = _lsr(raw64(seed, stream, start, n, device), 11)
    return (r.to(torch.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, stream: int, shape, device="cpu") -> torch.Tensor:
    """float64 N(0,1) samples via Box-Muller over consecutive uniform pairs."""
    n = int(math.prod(shape))
    m = (n + 1) // 2
    u = uniform(seed, stream, 2 * m, device).view(m, 2)
    r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
    t = (2.0 * math.pi) * u[:, 1]
    z = torch.stack((r * torch.cos(t), r * torch.sin(t)), dim=1).reshape(-1)[:n]
    return z.reshape(shape)


def randint_below(seed: int, stream: int, n: int, bound: int, device="cpu") -> torch.Tensor:
    """n integers uniform in [lo, bound) via floor(u * bound)."""
    return torch.floor(uniform(seed, stream, n, device) * bound).to(torch.int64)


def permutation(seed: int, stream: int, n: int, device="cpu") -> torch.Tensor:
    """A seeded permutation of 0..n-1 (argsort of distinct 64-bit keys)."""
    keys = raw64(seed, stream, 0, n, device)
    # ties between 64-bit keys are practically impossible; argsort is stable anyway
    return torch.argsort(keys, stable=True)


def quantize(x64: torch.Tensor, dtype: int, scale=1.0) -> torch.Tensor:
    """Round float64 values to the storage dtype (RNE).

    8-bit values are divided by ``scale`` (a number, or a tensor broadcast
    against x64) first and stored as OCP e4m3fn / e5m2 codes; the generator
    keeps |x/scale| <= 240 so no code saturates."""
    if dtype in EIGHT_BIT:
        y = (x64 / scale).to(torch.float32)
        return y.to(TORCH_DTYPE[dtype])
    return x64.to(TORCH_DTYPE[dtype])


def nan_fill(shape, dtype: int) -> torch.Tensor:
    """Storage-dtype tensor of NaN codes, used for page slots past a sequence's end."""
    if dtype in EIGHT_BIT:
        return torch.full(shape, 0x7F, dtype=torch.uint8).view(TORCH_DTYPE[dtype])
    return torch.full(shape, float("nan"), dtype=TORCH_DTYPE[dtype])


@dataclass
class Problem:
    """Host tensors of one attention call (storage dtypes, CPU)."""
    kind: str                     # "decode" | "prefill" | "blocksparse"
    batch: int
    q_rows: int                   # rows per sequence (decode R, prefill S_q)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: int
    q_dtype: int
    o_dtype: int
    seq_lens: torch.Tensor        # int32 [B]
    page_table: torch.Tensor      # int32 [B][stride]
    k_pool: torch.Tensor          # [num_pages][Hkv][16][d]   (storage dtype)
    v_pool: torch.Tensor          # [num_pages][Hkv][d][16]   (storage dtype, token-minor)
    q: torch.Tensor               # [B][q_rows][Hq][d]
    k_scale: float = 1.0
    v_scale: float = 1.0
    softmax_scale: float = 0.0
    sinks: Optional[torch.Tensor] = None      # float32 [Hq]
    mask: Optional[torch.Tensor] = None       # uint8 [B][mask_heads][nqb][nkb]
    mask_block: int = 128
    seed: int = 0
    meta: dict = field(default_factory=dict)
    rows_per_seq: Optional[torch.Tensor] = None   # int32 [B]: valid rows of each sequence
    k_vs: Optional[torch.Tensor] = None   # float32 [num_pages][Hkv][16]: per-vector K scales
    v_vs: Optional[torch.Tensor] = None   # float32 [num_pages][Hkv][16]: per-vector V scales


    @property
    def num_pages(self) -> int:
        return self.k_pool.shape[0]

    @property
    def page_table_stride(self) -> int:
        return self.page_table.shape[1]

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


def _vector_spread(seed, stream, shape, device):
    """Per-vector magnitude factors 2^U(-1, 1): token vectors of unequal size,
    so that per-vector scales differ from token to token."""
    n = int(math.prod(shape))
    return torch.exp2(2.0 * uniform(seed, stream, n, device) - 1.0).view(*shape, 1)


def _per_vector(x64: torch.Tensor, dtype: int):
    """Codes and float32 scales of vectors along the last axis: the generator's
    scale is amax / 240 (1 for an all-zero vector)."""
    amax = x64.abs().amax(dim=-1)
    sc = (amax / 240.0).to(torch.float32)
    sc = torch.where(sc == 0, torch.ones_like(sc), sc)
    return quantize(x64, dtype, sc.to(torch.float64).unsqueeze(-1)), sc


def _build_pool(seed, lens, stride, hkv, d, kv_dtype, pool_pages=None, device="cpu",
                k_scale=None, v_scale=None, extra_pages=0, vscales=False):
    """Generate logical K/V ~ N(0,1) per (sequence, kv head) and scatter them
    into a shuffled shared page pool.  Returns (k_pool, v_pool, page_table,
    k_scale, v_scale, k_vs, v_vs); with ``vscales`` (8-bit storage) every
    (token, head) vector is scaled by 2^U(-1,1) and stored with its own FP32
    scale in the pools k_vs / v_vs [pages][Hkv][16] (per-tensor scales 1),
    else k_vs = v_vs = None."""
    assert not vscales or kv_dtype in EIGHT_BIT
    B = len(lens)
    npages_b = [(int(L) + PAGE - 1) // PAGE for L in lens]
    total = sum(npages_b) + extra_pages
    perm = permutation(seed, 1, total, device)
    page_table = torch.zeros((B, stride), dtype=torch.int32, device=device)
    # unused table slots get random (valid) page ids: they must never matter
    if total:
        filler = randint_below(seed, 2, B * stride, total, device).to(torch.int32)
        page_table.copy_(filler.view(B, stride))
    off = 0
    for b in range(B):
        n = npages_b[b]
        assert n <= stride, "sequence longer than the page-table capacity"
        page_table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n

    tdt = TORCH_DTYPE[kv_dtype]
    k_pool = nan_fill((total, hkv, PAGE, d), kv_dtype).to(device)
    v_pool = nan_fill((total, hkv, d, PAGE), kv_dtype).to(device)
    k_vs = v_vs = None
    if vscales:
        # slots past a sequence's end hold NaN scales: they must never be used
        k_vs = torch.full((total, hkv, PAGE), float("nan"), dtype=torch.float32, device=device)
        v_vs = torch.full((total, hkv, PAGE), float("nan"), dtype=torch.float32, device=device)
        k_scale = v_scale = 1.0

    # 8-bit: per-tensor scale = amax / 240 over the whole logical K (resp. V);
    # a first pass finds the amax, the second regenerates and quantises
    if kv_dtype in EIGHT_BIT and (k_scale is None or v_scale is None):
        amax_k = amax_v = 0.0
        for b in range(B):
            L = int(lens[b])
            if L:
                amax_k = max(amax_k, float(normal(seed, 1000 + 2 * b, (hkv, L, d), device).abs().max()))
                amax_v = max(amax_v, float(normal(seed, 1001 + 2 * b, (hkv, L, d), device).abs().max()))
        k_scale = k_scale or float(torch.tensor(amax_k / 240.0, dtype=torch.float32))
        v_scale = v_scale or float(torch.tensor(amax_v / 240.0, dtype=torch.float32))
    k_scale = k_scale or 1.0
    v_scale = v_scale or 1.0

    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        kx = normal(seed, 1000 + 2 * b, (hkv, L, d), device)
        vx = normal(seed, 1001 + 2 * b, (hkv, L, d), device)
        n = npages_b[b]
        pad = n * PAGE - L
        ids = page_table[b, :n].to(torch.int64)
        if vscales:
            kq, ksc = _per_vector(kx * _vector_spread(seed, 2000 + 2 * b, (hkv, L), device), kv_dtype)
            vq, vsc = _per_vector(vx * _vector_spread(seed, 2001 + 2 * b, (hkv, L), device), kv_dtype)
            nanp = torch.full((hkv, pad), float("nan"), dtype=torch.float32, device=device)
            k_vs[ids] = torch.cat([ksc, nanp], dim=1).view(hkv, n, PAGE).permute(1, 0, 2)
            v_vs[ids] = torch.cat([vsc, nanp], dim=1).view(hkv, n, PAGE).permute(1, 0, 2)
        else:
            kq = quantize(kx, kv_dtype, k_scale)
            vq = quantize(vx, kv_dtype, v_scale)
        if pad:
            kq = torch.cat([kq, nan_fill((hkv, pad, d), kv_dtype).to(device)], dim=1)
            vq = torch.cat([vq, nan_fill((hkv, pad, d), kv_dtype).to(device)], dim=1)
        # [hkv][n*16][d] -> [n][hkv][16][d]; V pages are token-minor: [n][hkv][d][16]
        kt = kq.view(hkv, n, PAGE, d).permute(1, 0, 2, 3)
        vt = vq.view(hkv, n, PAGE, d).permute(1, 0, 3, 2)
        if kv_dtype in EIGHT_BIT:
            k_pool.view(torch.uint8)[ids] = kt.contiguous().view(torch.uint8)
            v_pool.view(torch.uint8)[ids] = vt.contiguous().view(torch.uint8)
        else:
            k_pool[ids] = kt.to(tdt)
            v_pool[ids] = vt.to(tdt)
    return k_pool, v_pool, page_table, k_scale, v_scale, k_vs, v_vs


def make_decode(seed, batch, num_q_heads, num_kv_heads, head_dim, lens, q_rows,
                kv_dtype=DT_BF16, q_dtype=None, o_dtype=None, stride=None, sinks=False,
                softmax_scale=0.0, device="cpu", extra_pages=0, rows_per_seq=None,
                vscales=False) -> Problem:
    """Paged decode / speculative-verify problem: ``q_rows`` rows per sequence
    sit at the last q_rows positions of each sequence (lens include them).
    With ``rows_per_seq`` (a list, each <= q_rows) sequence b has only its first
    rows_per_seq[b] rows, at its last rows_per_seq[b] positions.  ``vscales``
    (8-bit K/V): per-vector FP32 scales instead of per-tensor ones."""
    lens = [int(x) for x in lens]
    assert len(lens) == batch
    if stride is None:
        stride = max(1, max((L + PAGE - 1) // PAGE for L in lens))
    if q_dtype is None:
        q_dtype = DT_BF16 if kv_dtype in EIGHT_BIT else kv_dtype
    if o_dtype is None:
        o_dtype = q_dtype
    k_pool, v_pool, pt, ks, vs, kvs, vvs = _build_pool(seed, lens, stride, num_kv_heads, head_dim,
                                                       kv_dtype, device=device,
                                                       extra_pages=extra_pages, vscales=vscales)
    q = quantize(normal(seed, 3, (batch, q_rows, num_q_heads, head_dim), device), q_dtype)
    sk = None
    if sinks:
        sk = normal(seed, 4, (num_q_heads,), device).to(torch.float32)
    p = Problem("decode", batch, q_rows, num_q_heads, num_kv_heads, head_dim, kv_dtype,
                q_dtype, o_dtype, torch.tensor(lens, dtype=torch.int32, device=device), pt,
                k_pool, v_pool, q, ks, vs, softmax_scale, sk, None, 128, seed)
    p.k_vs, p.v_vs = kvs, vvs
    if rows_per_seq is not None:
        assert len(rows_per_seq) == batch and all(0 <= r <= q_rows for r in rows_per_seq)
        p.rows_per_seq = torch.tensor([int(r) for r in rows_per_seq], dtype=torch.int32,
                                      device=device)
    return p


def make_prefill(seed, batch, num_q_heads, num_kv_heads, head_dim, seq_len, q_rows=None,
                 kv_dtype=DT_BF16, sinks=True, lens=None, softmax_scale=0.0, device="cpu",
                 o_dtype=None, vscales=False) -> Problem:
    """Causal prefill problem: q_rows (default seq_len) query rows at the end
    of each sequence; all K/V (including the rows' own) are in the paged pool."""
    if lens is None:
        lens = [seq_len] * batch
    lens = [int(x) for x in lens]
    q_rows = seq_len if q_rows is None else q_rows
    stride = max(1, max((L + PAGE - 1) // PAGE for L in lens))
    q_dtype = DT_BF16 if kv_dtype in EIGHT_BIT + (DT_F32,) else kv_dtype
    if kv_dtype == DT_F32:
        q_dtype = DT_F32
    k_pool, v_pool, pt, ks, vs, kvs, vvs = _build_pool(seed, lens, stride, num_kv_heads, head_dim,
                                                       kv_dtype, device=device, vscales=vscales)
    q = quantize(normal(seed, 3, (batch, q_rows, num_q_heads, head_dim), device), q_dtype)
    sk = normal(seed, 4, (num_q_heads,), device).to(torch.float32) if sinks else None
    p = Problem("prefill", batch, q_rows, num_q_heads, num_kv_heads, head_dim, kv_dtype,
                q_dtype, o_dtype if o_dtype is not None else q_dtype,
                torch.tensor(lens, dtype=torch.int32, device=device), pt,
                k_pool, v_pool, q, ks, vs, softmax_scale, sk, None, 128, seed)
    p.k_vs, p.v_vs = kvs, vvs
    return p


def flashprefill_mask(seed, batch, mask_heads, n_blocks, keep_prob=0.1, device="cpu"):
    """Block mask [B][mask_heads][nqb][nkb] (uint8, 1 = keep): each query block
    keeps KV block 0, its diagonal block and a Bernoulli(keep_prob) draw of
    every block strictly between them.  Blocks above the diagonal are 0."""
    u = uniform(seed, 5, batch * mask_heads * n_blocks * n_blocks, device)
    u = u.view(batch, mask_heads, n_blocks, n_blocks)
    m = (u < keep_prob).to(torch.uint8)
    qb = torch.arange(n_blocks, device=device).view(-1, 1)
    kb = torch.arange(n_blocks, device=device).view(1, -1)
    m = torch.where(kb > qb, torch.zeros_like(m), m)
    m = torch.where((kb == 0) | (kb == qb), torch.ones_like(m), m)
    return m.contiguous()


def make_blocksparse(seed, batch, num_q_heads, num_kv_heads, head_dim, seq_len,
                     mask_block=128, mask_heads=1, keep_prob=0.1, sinks=False,
                     kv_dtype=DT_BF16, device="cpu", mask=None, vscales=False) -> Problem:
    p = make_prefill(seed, batch, num_q_heads, num_kv_heads, head_dim, seq_len,
                     kv_dtype=kv_dtype, sinks=sinks, device=device, vscales=vscales)
    nb = (seq_len + mask_block - 1) // mask_block
    p.kind = "blocksparse"
    p.mask = mask if mask is not None else flashprefill_mask(seed, batch, mask_heads, nb,
                                                             keep_prob, device)
    p.mask_block = mask_block
    return p


# --- the five workloads of the path, at their stated sizes ------------------------

def config1(seed=101):
    """Tiny paged decode: 1 sequence, 4 q heads, 1 kv head, d=64, 256 tokens,
    FP32 Q/K/V, one row, scale 1/8, no sink."""
    return make_decode(seed, 1, 4, 1, 64, [256], 1, kv_dtype=DT_F32, q_dtype=DT_F32,
                       o_dtype=DT_F32, softmax_scale=1.0 / 8.0)


def config2_lens(seed=202, batch=16, lo=8192, hi=16384):
    return [int(x) for x in (lo + randint_below(seed, 6, batch, hi - lo + 1))]


def config2(seed=202, q_rows=1, lens=None, batch=16, device="cpu"):
    """Paged decode / verify: B=16, Hq=32, Hkv=8, d=128, BF16, table stride 1024."""
    if lens is None:
        lens = config2_lens(seed, batch)
    return make_decode(seed, batch, 32, 8, 128, lens, q_rows, kv_dtype=DT_BF16,
                       stride=1024, device=device)


def config3(seed=303, batch=4, ctx=65536, device="cpu", kv_dtype=DT_FP8, vscales=False):
    """FP8-e4m3 long decode: B=4, Hq=32, Hkv=8, d=128, 64K context, 4 rows (also
    with e5m2 storage or per-vector scales)."""
    return make_decode(seed, batch, 32, 8, 128, [ctx] * batch, 4, kv_dtype=kv_dtype,
                       q_dtype=DT_BF16, o_dtype=DT_BF16, stride=(ctx + 15) // 16, device=device,
                       vscales=vscales)


def config4(seed=404, seq_len=8192, batch=16, device="cpu", kv_dtype=DT_BF16, vscales=False):
    """Causal prefill with sinks: Hq=64, Hkv=8, d=64, BF16 (or 8-bit) K/V, scale 1/8."""
    return make_prefill(seed, batch, 64, 8, 64, seq_len, sinks=True, softmax_scale=0.125,
                        device=device, kv_dtype=kv_dtype, vscales=vscales)


def config5(seed=505, seq_len=32768, device="cpu"):
    """Block-sparse long prefill: 1 x 32K, Hq=32, Hkv=8, d=128, 128-token blocks."""
    return make_blocksparse(seed, 1, 32, 8, 128, seq_len, mask_block=128, mask_heads=1,
                            keep_prob=0.1, device=device)


# --- helpers used by tests to read back or overwrite the logical K/V ----------------

def logical_kv_codes(p: Problem, b: int):
    """The quantised logical K and V codes of sequence b as stored: [Hkv][L][d]
    tensors of the storage dtype, read back out of the page pool."""
    L = int(p.seq_lens[b])
    n = (L + PAGE - 1) // PAGE
    ids = p.page_table[b, :n].to(torch.int64).cpu()
    kp, vp = p.k_pool.cpu(), p.v_pool.cpu()
    if p.kv_dtype in EIGHT_BIT:
        kp, vp = kp.view(torch.uint8), vp.view(torch.uint8)
    k = kp[ids].permute(1, 0, 2, 3).reshape(p.num_kv_heads, n * PAGE, p.head_dim)[:, :L]
    v = vp[ids].permute(1, 0, 3, 2).reshape(p.num_kv_heads, n * PAGE, p.head_dim)[:, :L]
    if p.kv_dtype in EIGHT_BIT:
        k, v = k.view(TORCH_DTYPE[p.kv_dtype]), v.view(TORCH_DTYPE[p.kv_dtype])
    return k.contiguous(), v.contiguous()


def logical_vscales(p: Problem, b: int):
    """The per-vector K and V scales of sequence b as stored: float32 [Hkv][L]."""
    L = int(p.seq_lens[b])
    n = (L + PAGE - 1) // PAGE
    ids = p.page_table[b, :n].to(torch.int64).cpu()
    ks = p.k_vs.cpu()[ids].permute(1, 0, 2).reshape(p.num_kv_heads, n * PAGE)[:, :L]
    vs = p.v_vs.cpu()[ids].permute(1, 0, 2).reshape(p.num_kv_heads, n * PAGE)[:, :L]
    return ks.contiguous(), vs.contiguous()


def store_logical_kv(p: Problem, b: int, g: int, k=None, v=None):
    """Overwrite the logical K and/or V ([L][d], storage dtype) of (b, g) in the pool."""
    L = int(p.seq_lens[b])
    n = (L + PAGE - 1) // PAGE
    ids = p.page_table[b, :n].to(torch.int64)
    for src, pool, tr in ((k, p.k_pool, False), (v, p.v_pool, True)):
        if src is None:
            continue
        src = src.to(pool.dtype) if pool.dtype not in (torch.float8_e4m3fn, torch.float8_e5m2) else src
        for pg in range(n):
            t0, t1 = pg * PAGE, min(L, pg * PAGE + PAGE)
            blk = src[t0:t1]
            if tr:
                pool[ids[pg], g, :, : t1 - t0] = blk.transpose(0, 1)
            else:
                pool[ids[pg], g, : t1 - t0, :] = blk


_CODE_VIEW = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16,
              torch.float8_e4m3fn: torch.uint8, torch.float8_e5m2: torch.uint8}
_CODE_NP = {torch.float32: "uint32", torch.float16: "uint16", torch.bfloat16: "uint16",
            torch.float8_e4m3fn: "uint8", torch.float8_e5m2: "uint8"}


def pool_codes(pool: torch.Tensor):
    """The raw storage codes of a K or V pool as a numpy array of unsigned ints."""
    t = pool.detach().cpu().contiguous()
    return t.view(_CODE_VIEW[t.dtype]).numpy().view(_CODE_NP[t.dtype])


def with_pool_codes(p: Problem, k_codes, v_codes) -> Problem:
    """A copy of p whose K/V pools hold the given raw storage codes."""
    import copy
    import numpy as np
    q = copy.copy(p)
    dt = p.k_pool.dtype
    view = _CODE_VIEW[dt]
    conv = lambda c: torch.from_numpy(np.ascontiguousarray(c).view(
        {torch.int32: np.int32, torch.int16: np.int16, torch.uint8: np.uint8}[view])).view(dt)
    q.k_pool, q.v_pool = conv(k_codes), conv(v_codes)
    return q


def append_rows(seed: int, batch: int, n_new: int, num_kv_heads: int, head_dim: int,
                dtype=torch.bfloat16, device="cpu"):
    """New K and V rows [B][n_new][Hkv][d] ~ N(0,1), rounded once to `dtype`."""
    shape = (batch, n_new, num_kv_heads, head_dim)
    k = normal(seed, 0, shape).to(dtype)
    v = normal(seed, 1, shape).to(dtype)
    return k.to(device), v.to(device)
