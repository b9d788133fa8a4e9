"""Byte and FLOP accounting for the paged attention calls.

These closed forms give the *algorithmic* traffic and work of one call
(what the method must read and write at least once), used to express
measured times as a fraction of the MI355X roofline.
"""
from __future__ import annotations

ELT_BYTES = {0: 4, 1: 2, 2: 2, 3: 1, 4: 1}   # f32, f16, bf16, fp8-e4m3, bf8-e5m2
PAGE = 16


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype: int,
                       per_vector_scales: bool = False) -> int:
    """K+V bytes one token occupies across all layers.

    With ``per_vector_scales`` every (layer, head, K-or-V) vector carries one
    FP32 scale, the FP8 storage format of the Geramy/LSE README's K/V storage
    table (33,280 B per token for 16 layers x 4 heads x 256)."""
    vecs = layers * kv_heads * 2
    b = vecs * head_dim * ELT_BYTES[dtype]
    if per_vector_scales:
        b += vecs * 4
    return b


def decode_bytes(lens, q_rows, num_q_heads, num_kv_heads, head_dim, kv_dtype, q_dtype,
                 o_dtype, per_vector_scales: bool = False) -> int:
    """Algorithmic HBM bytes of one paged decode call: every live K/V element
    once (with its vector's FP32 scale where the cache has per-vector scales),
    the query rows, the outputs and the used page-table entries."""
    per_vec = head_dim * ELT_BYTES[kv_dtype] + (4 if per_vector_scales else 0)
    kv = sum(int(L) for L in lens) * num_kv_heads * per_vec * 2
    B = len(lens)
    q = B * q_rows * num_q_heads * head_dim * ELT_BYTES[q_dtype]
    o = B * q_rows * num_q_heads * head_dim * ELT_BYTES[o_dtype]
    pt = sum((int(L) + PAGE - 1) // PAGE for L in lens) * 4
    return kv + q + o + pt


def causal_pairs(q_rows: int, seq_len: int) -> int:
    """(query, key) pairs of causal attention of q_rows rows ending at seq_len."""
    total = 0
    n0 = seq_len - q_rows
    # row i sees n0 + i + 1 keys
    return q_rows * (n0 + 1) + q_rows * (q_rows - 1) // 2 if q_rows > 0 else total


def attention_flops(pairs: int, num_q_heads: int, head_dim: int, batch: int = 1) -> int:
    """2 flops per multiply-add, QK^T and PV each head_dim MACs per pair."""
    return 4 * batch * num_q_heads * head_dim * pairs


def mask_pairs(mask_row_blocks, seq_len: int, block: int) -> int:
    """Allowed causal pairs under a block mask (one mask head), exact count.

    ``mask_row_blocks[qb]`` lists the kept key blocks of query block qb."""
    total = 0
    for qb, kbs in enumerate(mask_row_blocks):
        q0, q1 = qb * block, min(seq_len, qb * block + block)
        for kb in kbs:
            k0, k1 = kb * block, min(seq_len, kb * block + block)
            if kb < qb:
                total += (q1 - q0) * (k1 - k0)
            elif kb == qb:
                n = q1 - q0
                total += n * (n + 1) // 2
    return total
