"""Pins of the FP64 oracle to facts outside itself.

Each test checks the oracle against something the pages or mathematics fix:
independent decodings of every storage code, a bit-exact gather back to the
generator's logical arrays, brute-force softmax in extended precision on tiny
inputs, closed forms (Q = 0, one-hot V, constant V, a single key, constant
scores), and invariants (sink = -inf, page permutation, split + merge,
causal alignment of prefill and verify rows, all-ones and block-diagonal
masks, MHA replication of KV heads).  A dropped term, a wrong sign or index
or a transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import DT_BF16, DT_BF8, DT_F16, DT_F32, DT_FP8, PAGE


# ---------------------------------------------------------------- storage codes

def test_bf16_every_code():
    codes = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_codes(DT_BF16, codes)
    # independent route: a bf16 code is the top half of an IEEE float32
    ref = (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_every_code():
    codes = np.arange(65536, dtype=np.uint16)
    got = oracle.decode_codes(DT_F16, codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_codes(DT_FP8, codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]          # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # special values of the OCP e4m3fn format
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0           # largest finite
    assert got[0x01] == 2.0 ** -9                                # smallest subnormal
    assert got[0x08] == 2.0 ** -6                                # smallest normal
    assert got[0x00] == 0.0 and math.copysign(1, got[0x80]) == -1.0
    assert got[0x38] == 1.0


def test_e5m2_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_codes(DT_BF8, codes)
    # independent route: an e5m2 code is the top byte of an IEEE binary16
    ref = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 6                                       # S.11111.{01,10,11}
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    tref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(got[~nan], tref[~nan])
    assert got[0x7B] == 57344.0 and got[0x7C] == math.inf and got[0xFC] == -math.inf
    assert got[0x01] == 2.0 ** -16 and got[0x04] == 2.0 ** -14 and got[0x3C] == 1.0


def test_f32_codes_roundtrip():
    x = synth.normal(9, 0, (1000,)).to(torch.float32)
    got = oracle.decode_codes(DT_F32, x.numpy().view(np.uint32))
    assert np.array_equal(got, x.to(torch.float64).numpy())


# ---------------------------------------------------------------- paged gather

@pytest.mark.parametrize("dtype,vscales", [(DT_F32, False), (DT_F16, False), (DT_BF16, False),
                                           (DT_FP8, False), (DT_BF8, False), (DT_FP8, True),
                                           (DT_BF8, True)])
def test_gather_bit_exact(dtype, vscales):
    p = synth.make_decode(11, 3, 4, 2, 64, [37, 16, 5], 1, kv_dtype=dtype, stride=4,
                          vscales=vscales)
    for b in range(p.batch):
        kc, vc = synth.logical_kv_codes(p, b)
        if vscales:
            ks, vs = (t.to(torch.float64).numpy()[..., None] for t in synth.logical_vscales(p, b))
            assert np.all(np.isfinite(ks)) and np.all(np.isfinite(vs))
        for g in range(p.num_kv_heads):
            k, v = oracle.gather(p, b, g)
            kref = kc[g].to(torch.float64).numpy() * p.k_scale
            vref = vc[g].to(torch.float64).numpy() * p.v_scale
            if vscales:      # code * per-vector scale: exact in double precision
                kref, vref = kref * ks[g], vref * vs[g]
            assert np.array_equal(k, kref) and np.array_equal(v, vref)


def test_generator_logical_values_match_the_pool():
    """The pool holds the generator's own N(0,1) draws rounded once."""
    p = synth.make_decode(12, 2, 4, 2, 64, [20, 33], 1, kv_dtype=DT_BF16)
    for b in range(2):
        kc, vc = synth.logical_kv_codes(p, b)
        L = int(p.seq_lens[b])
        kref = synth.normal(12, 1000 + 2 * b, (2, L, 64)).to(torch.bfloat16)
        vref = synth.normal(12, 1001 + 2 * b, (2, L, 64)).to(torch.bfloat16)
        assert torch.equal(kc, kref) and torch.equal(vc, vref)


# ---------------------------------------------------------------- brute force

def _brute(p, b, i, h):
    """softmax by the definition in extended precision, no max shift."""
    G = p.num_q_heads // p.num_kv_heads
    g = h // G
    L = int(p.seq_lens[b])
    pos = L - p.q_rows + i
    kc, vc = synth.logical_kv_codes(p, b)
    K = kc[g].to(torch.float64).numpy().astype(np.longdouble) * p.k_scale
    V = vc[g].to(torch.float64).numpy().astype(np.longdouble) * p.v_scale
    if p.k_vs is not None:
        ks, vs = synth.logical_vscales(p, b)
        K = K * ks[g].to(torch.float64).numpy().astype(np.longdouble)[:, None]
        V = V * vs[g].to(torch.float64).numpy().astype(np.longdouble)[:, None]
    q = p.q[b, i, h].to(torch.float64).numpy().astype(np.longdouble)
    allowed = []
    for j in range(L):
        ok = j <= pos
        if ok and p.mask is not None:
            qb, kb = pos // p.mask_block, j // p.mask_block
            mh = 0 if p.mask.shape[1] == 1 else g
            ok = qb < p.mask.shape[2] and kb < p.mask.shape[3] and bool(p.mask[b, mh, qb, kb])
        if ok:
            allowed.append(j)
    w = np.array([np.exp(np.longdouble(p.scale) * np.dot(q, K[j])) for j in allowed],
                 dtype=np.longdouble)
    sink = np.exp(np.longdouble(float(p.sinks[h]))) if p.sinks is not None else np.longdouble(0)
    Z = w.sum() + sink
    if Z == 0:
        return np.zeros(p.head_dim), -math.inf
    o = (w[:, None] * V[allowed]).sum(axis=0) / Z if allowed else np.zeros(p.head_dim)
    return o.astype(np.float64), float(np.log(Z))


@pytest.mark.parametrize("kv_dtype,vscales", [(DT_F32, False), (DT_BF16, False), (DT_FP8, False),
                                              (DT_BF8, False), (DT_FP8, True), (DT_BF8, True)])
@pytest.mark.parametrize("sinks", [False, True])
def test_brute_force_decode(kv_dtype, vscales, sinks):
    p = synth.make_decode(21, 2, 4, 2, 8, [37, 50], 3, kv_dtype=kv_dtype, sinks=sinks,
                          softmax_scale=0.3, vscales=vscales)
    o, lse = oracle.attend_full(p)
    for b in range(2):
        for i in range(3):
            for h in range(4):
                ob, lb = _brute(p, b, i, h)
                assert np.max(np.abs(o[b, i, h] - ob)) <= 1e-13
                assert abs(lse[b, h, i] - lb) <= 1e-13


def test_brute_force_prefill_with_random_mask():
    p = synth.make_blocksparse(22, 2, 4, 2, 8, 40, mask_block=8, mask_heads=2, keep_prob=0.5,
                               sinks=True)
    # an asymmetric random mask (also above the diagonal, which must be ignored)
    u = synth.uniform(22, 77, p.mask.numel()).view(p.mask.shape)
    p.mask = (u < 0.6).to(torch.uint8)
    o, lse = oracle.attend_full(p)
    for b in range(2):
        for i in range(0, 40, 3):
            for h in range(4):
                ob, lb = _brute(p, b, i, h)
                assert np.max(np.abs(o[b, i, h] - ob)) <= 1e-13
                assert abs(lse[b, h, i] - lb) <= 1e-13 or (lse[b, h, i] == lb == -math.inf)


# ---------------------------------------------------------------- closed forms

def _qzero(p):
    p.q = torch.zeros_like(p.q)
    return p


def test_q_zero_gives_mean_of_values_and_log_n():
    p = _qzero(synth.make_decode(31, 2, 4, 1, 16, [24, 9], 1, kv_dtype=DT_F32))
    o, lse = oracle.attend_full(p)
    for b in range(2):
        L = int(p.seq_lens[b])
        k, v = oracle.gather(p, b, 0)
        for h in range(4):
            assert np.allclose(o[b, 0, h], v.mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[b, h, 0] - math.log(L)) <= 1e-14


def test_q_zero_with_sink_closed_form():
    p = _qzero(synth.make_decode(32, 1, 4, 1, 16, [24], 1, kv_dtype=DT_F32, sinks=True))
    o, lse = oracle.attend_full(p)
    k, v = oracle.gather(p, 0, 0)
    for h in range(4):
        s = float(p.sinks[h])
        ref = v.sum(axis=0) / (24 + math.exp(s))
        assert np.allclose(o[0, 0, h], ref, rtol=0, atol=1e-14)
        assert abs(lse[0, h, 0] - math.log(24 + math.exp(s))) <= 1e-13


def test_one_hot_values_return_probabilities_that_sum_to_one():
    """V_j = e_j makes o the probability vector; with the sink's share
    exp(sink - lse) the probabilities sum to one."""
    d, L = 32, 29
    p = synth.make_decode(33, 1, 2, 1, d, [L], 1, kv_dtype=DT_F32, sinks=True)
    synth.store_logical_kv(p, 0, 0, v=torch.eye(L, d, dtype=torch.float32))
    o, lse = oracle.attend_full(p)
    kc, _ = synth.logical_kv_codes(p, 0)
    K = kc[0].to(torch.float64).numpy()
    for h in range(2):
        q = p.q[0, 0, h].to(torch.float64).numpy()
        s = p.scale * (K @ q)
        sink = float(p.sinks[h])
        prob = np.exp(s - lse[0, h, 0])
        assert np.allclose(o[0, 0, h][:L], prob, rtol=1e-13, atol=1e-15)
        assert abs(o[0, 0, h][:L].sum() + math.exp(sink - lse[0, h, 0]) - 1.0) <= 1e-12


def test_constant_values_scale_by_one_minus_sink_share():
    d, L = 16, 40
    p = synth.make_decode(34, 1, 4, 1, d, [L], 1, kv_dtype=DT_F32, sinks=True)
    c = torch.linspace(-2, 3, d, dtype=torch.float32)
    synth.store_logical_kv(p, 0, 0, v=c.expand(L, d).clone())
    o, lse = oracle.attend_full(p)
    for h in range(4):
        p_sink = math.exp(float(p.sinks[h]) - lse[0, h, 0])
        assert np.allclose(o[0, 0, h], c.double().numpy() * (1 - p_sink), rtol=0, atol=1e-13)


def test_single_key_with_sink_is_a_sigmoid():
    p = synth.make_decode(35, 1, 4, 1, 16, [1], 1, kv_dtype=DT_F32, sinks=True)
    o, lse = oracle.attend_full(p)
    k, v = oracle.gather(p, 0, 0)
    for h in range(4):
        s0 = p.scale * float(np.dot(p.q[0, 0, h].double().numpy(), k[0]))
        sig = 1.0 / (1.0 + math.exp(float(p.sinks[h]) - s0))
        assert np.allclose(o[0, 0, h], v[0] * sig, rtol=0, atol=1e-14)


def test_empty_rows():
    """No allowed key: o = 0 and lse = sink (or -inf without a sink)."""
    p = synth.make_decode(36, 2, 4, 2, 16, [0, 3], 4, kv_dtype=DT_BF16, sinks=True)
    o, lse = oracle.attend_full(p)
    assert np.all(o[0] == 0)
    assert np.allclose(lse[0], p.sinks.double().numpy()[:, None].repeat(4, axis=1))
    # sequence 1 has 3 keys and 4 rows: row 0 sits at position -1
    assert np.all(o[1, 0] == 0)
    p.sinks = None
    o, lse = oracle.attend_full(p)
    assert np.all(np.isneginf(lse[0])) and np.all(o[0] == 0)


# ---------------------------------------------------------------- invariants

def test_sink_minus_inf_equals_no_sink():
    p = synth.make_decode(41, 2, 8, 2, 32, [70, 33], 2, kv_dtype=DT_BF16)
    o0, l0 = oracle.attend_full(p)
    p.sinks = torch.full((8,), -math.inf, dtype=torch.float32)
    o1, l1 = oracle.attend_full(p)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_page_table_permutation_invariance():
    p = synth.make_decode(42, 2, 4, 2, 32, [70, 33], 2, kv_dtype=DT_BF16, extra_pages=5)
    o0, l0 = oracle.attend_full(p)
    perm = synth.permutation(42, 99, p.num_pages)            # new page id of page k
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(p.num_pages)
    p.k_pool = p.k_pool[inv].contiguous()
    p.v_pool = p.v_pool[inv].contiguous()
    p.page_table = perm[p.page_table.long()].to(torch.int32)
    o1, l1 = oracle.attend_full(p)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("cuts", [[0, 300], [0, 7, 7, 100, 300], [0, 1, 64, 65, 128, 250, 300]])
def test_split_and_merge_equals_unsplit(cuts):
    p = synth.make_decode(43, 1, 4, 1, 32, [300], 3, kv_dtype=DT_BF16, sinks=True)
    o, lse = oracle.attend_full(p)
    for i in range(3):
        for h in range(4):
            parts = [oracle.attend_partial(p, 0, i, h, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
            om, lm = oracle.merge(np.stack([x[0] for x in parts]), [x[1] for x in parts],
                                  [x[2] for x in parts], float(p.sinks[h]))
            assert np.allclose(om, o[0, i, h], rtol=1e-12, atol=1e-14)
            assert abs(lm - lse[0, h, i]) <= 1e-12 * max(1.0, abs(lm))


def test_prefill_row_equals_single_row_decode():
    p = synth.make_prefill(44, 1, 4, 2, 16, 37, kv_dtype=DT_BF16, sinks=True)
    o, lse = oracle.attend_full(p)
    for i in [0, 1, 15, 16, 36]:
        d = synth.make_decode(44, 1, 4, 2, 16, [37], 1, kv_dtype=DT_BF16)
        d.k_pool, d.v_pool, d.page_table, d.sinks = p.k_pool, p.v_pool, p.page_table, p.sinks
        d.seq_lens = torch.tensor([i + 1], dtype=torch.int32)
        d.q = p.q[:, i:i + 1].clone()
        od, ld = oracle.attend_full(d)
        assert np.array_equal(od[0, 0], o[0, i]) and np.array_equal(ld[0, :, 0], lse[0, :, i])


def test_verify_row_equals_decode_at_its_position():
    R, L = 8, 53
    p = synth.make_decode(45, 1, 8, 2, 16, [L], R, kv_dtype=DT_BF16, sinks=True)
    o, lse = oracle.attend_full(p)
    for r in range(R):
        d = synth.make_decode(45, 1, 8, 2, 16, [L], 1, kv_dtype=DT_BF16)
        d.k_pool, d.v_pool, d.page_table, d.sinks = p.k_pool, p.v_pool, p.page_table, p.sinks
        d.seq_lens = torch.tensor([L - R + r + 1], dtype=torch.int32)
        d.q = p.q[:, r:r + 1].clone()
        od, ld = oracle.attend_full(d)
        assert np.array_equal(od[0, 0], o[0, r]) and np.array_equal(ld[0, :, 0], lse[0, :, r])


def test_ragged_rows_equal_decode_at_their_positions():
    """Rows per sequence vary: row i of sequence b (of r_b rows) is the
    single-row decode at position L_b - r_b + i; rows i >= r_b do not exist."""
    R, lens, rps = 4, [53, 40, 17, 30], [4, 1, 3, 0]
    p = synth.make_decode(47, 4, 8, 2, 16, lens, R, kv_dtype=DT_BF16, sinks=True, rows_per_seq=rps)
    o, lse = oracle.attend_full(p)
    for b, (L, rb) in enumerate(zip(lens, rps)):
        for i in range(R):
            if i >= rb:
                assert np.all(np.isnan(o[b, i])) and np.all(np.isnan(lse[b, :, i]))
                continue
            d = synth.make_decode(47, 1, 8, 2, 16, [L], 1, kv_dtype=DT_BF16)
            d.k_pool, d.v_pool, d.sinks = p.k_pool, p.v_pool, p.sinks
            d.page_table = p.page_table[b:b + 1].clone()
            d.seq_lens = torch.tensor([L - rb + i + 1], dtype=torch.int32)
            d.q = p.q[b:b + 1, i:i + 1].clone()
            od, ld = oracle.attend_full(d)
            assert np.array_equal(od[0, 0], o[b, i]) and np.array_equal(ld[0, :, 0], lse[b, :, i])


def test_all_ones_mask_equals_dense_causal():
    p = synth.make_blocksparse(46, 2, 4, 2, 16, 70, mask_block=16, sinks=True)
    p.mask = torch.ones_like(p.mask)
    o1, l1 = oracle.attend_full(p)
    p.mask = None
    o0, l0 = oracle.attend_full(p)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_diagonal_mask_is_block_local_causal_attention():
    blk, S = 16, 64
    p = synth.make_blocksparse(47, 1, 4, 2, 16, S, mask_block=blk)
    nb = S // blk
    p.mask = torch.eye(nb, dtype=torch.uint8).view(1, 1, nb, nb).clone()
    o, lse = oracle.attend_full(p)
    kc, vc = synth.logical_kv_codes(p, 0)
    for h in range(4):
        K = kc[h // 2].double().numpy()
        V = vc[h // 2].double().numpy()
        for i in range(S):
            q = p.q[0, i, h].double().numpy()
            j0 = (i // blk) * blk
            s = p.scale * (K[j0:i + 1] @ q)
            w = np.exp(s - s.max())
            ref = (w[:, None] * V[j0:i + 1]).sum(0) / w.sum()
            assert np.allclose(o[0, i, h], ref, rtol=0, atol=1e-13)


def test_mha_replication_of_kv_heads():
    """Replicating every KV head G times (Hkv = Hq) must not change the output."""
    Hq, Hkv, G = 8, 2, 4
    p = synth.make_decode(48, 2, Hq, Hkv, 16, [40, 21], 2, kv_dtype=DT_BF16, sinks=True)
    o0, l0 = oracle.attend_full(p)
    p.k_pool = p.k_pool.repeat_interleave(G, dim=1).contiguous()
    p.v_pool = p.v_pool.repeat_interleave(G, dim=1).contiguous()
    p.num_kv_heads = Hq
    o1, l1 = oracle.attend_full(p)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_pages_past_the_end_are_ignored():
    p = synth.make_decode(49, 1, 4, 1, 16, [37], 1, kv_dtype=DT_BF16, stride=8, extra_pages=4)
    o0, l0 = oracle.attend_full(p)
    p.page_table[0, 3:] = torch.tensor([40, 41, 3, 0, 1], dtype=torch.int32) % p.num_pages
    o1, l1 = oracle.attend_full(p)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


# ---------------------------------------------------------------- corners of the definition

@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_lengths_beyond_capacity_count_as_the_capacity(kind):
    """A seq_lens entry above the page table's capacity (stride * 16) counts as
    the capacity: the rows sit at the capacity's last positions and see only
    the keys the table addresses.  Brute force over the first `cap` keys."""
    stride = 3
    cap = stride * PAGE
    if kind == "decode":
        p = synth.make_decode(71, 2, 4, 2, 8, [cap, cap], 3, kv_dtype=DT_BF16, stride=stride,
                              sinks=True, softmax_scale=0.4)
    else:
        p = synth.make_prefill(72, 2, 4, 2, 8, cap, kv_dtype=DT_BF16, sinks=True,
                               softmax_scale=0.4)
    ref = {(b, i, h): _brute(p, b, i, h) for b in range(2) for i in range(p.q_rows)
           for h in range(4)}
    p.seq_lens = torch.tensor([cap + 9, 2 ** 30], dtype=torch.int32)
    o, lse = oracle.attend_full(p)
    for (b, i, h), (ob, lb) in ref.items():
        assert np.max(np.abs(o[b, i, h] - ob)) <= 1e-13
        assert abs(lse[b, h, i] - lb) <= 1e-13
    # the gather stops at the capacity too
    k, v = oracle.gather(p, 1, 1)
    assert k.shape == (cap, 8) and v.shape == (cap, 8)


def test_mask_entries_outside_its_extent_count_as_zero():
    """A block mask with fewer query and key blocks than the sequence has: the
    missing entries drop their keys, exactly as explicit zeros would.  Brute
    force on the zero-padded mask (whose extent covers every block)."""
    S, blk = 40, 8
    p = synth.make_blocksparse(73, 2, 4, 2, 8, S, mask_block=blk, mask_heads=2, sinks=True)
    nb = S // blk
    u = synth.uniform(73, 78, 2 * 2 * nb * nb).view(2, 2, nb, nb)
    full = (u < 0.7).to(torch.uint8)
    small = full[:, :, :3, :2].contiguous()           # 3 of 5 query blocks, 2 of 5 key blocks
    padded = torch.zeros_like(full)
    padded[:, :, :3, :2] = small
    p.mask = padded
    ref = {(b, i, h): _brute(p, b, i, h) for b in range(2) for i in range(S) for h in range(4)}
    p.mask = small
    o, lse = oracle.attend_full(p)
    for (b, i, h), (ob, lb) in ref.items():
        assert np.max(np.abs(o[b, i, h] - ob)) <= 1e-13
        assert abs(lse[b, h, i] - lb) <= 1e-13
    # rows of query blocks past the mask keep no key: o = 0, lse = the sink
    assert np.all(o[:, 3 * blk:] == 0)
    assert np.allclose(lse[:, :, 3 * blk:], p.sinks.double().numpy()[None, :, None])
