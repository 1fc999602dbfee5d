"""Host-side policies of the Python binding (no GPU needed): the MLA decode's default split
size, pinned to the values its rule gives by hand."""
import pytest

import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs


def test_mla_default_split_mla_decode_b64_at_256_cus():
    """64 sequences of 1-4K keys on 256 compute units: with the lengths, the shortest
    16-key multiple whose items sum(ceil(len / split)) fit 256 workgroups is 752 keys
    (252 items; 736 keys would need 257)."""
    lens = inputs.mla_decode_b64().kv_lens()
    B, mx, tot = len(lens), max(lens), sum(lens)
    split = pkv.mla_decode_default_split(B, mx, tot, kv_lens=lens, cus=256)
    assert split == 752
    items = lambda s: sum(-(-x // s) for x in lens)
    assert items(752) <= 256 < items(736)
    # without the lengths: the shorter of max_kv / (CUs // B) and total / (CUs - B), in 16s
    no_lens = pkv.mla_decode_default_split(B, mx, tot, cus=256)
    want = min(-(-mx // (256 // B)), -(-tot // (256 - B)))
    assert no_lens == -(-want // 16) * 16


@pytest.mark.parametrize("B,length,want", [
    (256, 1000, 1008),  # one item per sequence: 63 sixteens, the smallest that keeps 1000 keys in one split
    (257, 1000, 1008),  # more batches than the packing handles: max_kv / max(1, CUs // B)
    (1, 100000, 400),   # one sequence: 100000 / 256 keys, rounded up to a multiple of 16
    (4, 0, 16),         # empty batch: the 16-key minimum
])
def test_mla_default_split_edges(B, length, want):
    lens = [length] * B
    assert pkv.mla_decode_default_split(B, length, length * B, kv_lens=lens, cus=256) == want
