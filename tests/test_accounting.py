"""Host-side byte/FLOP accounting pinned to the pages' KV-bytes table."""
import os

import pytest

from paged_gqa_attention_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes_per_token.txt")
DT = {"fp32": 0, "fp16": 1, "bf16": 2, "fp8": 3, "bf8": 4}


def _rows():
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, bpt, gib = line.split()
                yield name, int(bpt), float(gib)


@pytest.mark.parametrize("name,bpt,gib", list(_rows()))
def test_kv_bytes_table(name, bpt, gib):
    got = acc.kv_bytes_per_token(16, 4, 256, DT[name], per_vector_scales=name in ("fp8", "bf8"))
    assert got == bpt
    assert round(got * 32768 / 2 ** 30, 2) == gib


def test_causal_pairs():
    assert acc.causal_pairs(8192, 8192) == 8192 * 8193 // 2
    assert acc.causal_pairs(1, 100) == 100
    assert acc.causal_pairs(4, 10) == 7 + 8 + 9 + 10


def test_mask_pairs_full_equals_causal():
    S, blk = 1000, 128
    nb = (S + blk - 1) // blk
    rows = [list(range(qb + 1)) for qb in range(nb)]
    assert acc.mask_pairs(rows, S, blk) == acc.causal_pairs(S, S)


def test_decode_bytes_headline():
    # 16 x 16K tokens x 8 KV heads x 128 x bf16 x (K, V) = 1 GiB
    b = acc.decode_bytes([16384] * 16, 1, 32, 8, 128, 2, 2, 2)
    assert b - 2 ** 30 == 2 * 16 * 32 * 128 * 2 + 16 * 1024 * 4


def test_decode_bytes_per_vector_scales():
    # every live (token, head) carries one FP32 scale for K and one for V
    plain = acc.decode_bytes([1000, 37], 4, 32, 8, 128, 3, 2, 2)
    scaled = acc.decode_bytes([1000, 37], 4, 32, 8, 128, 3, 2, 2, per_vector_scales=True)
    assert scaled - plain == 1037 * 8 * 2 * 4
    assert acc.decode_bytes([16], 1, 1, 1, 64, 4, 2, 2) == 16 * 64 * 2 + 2 * 64 * 2 + 4
