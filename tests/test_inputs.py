"""Seeded input generators: reproducible, well-formed page tables, exact layout round trips."""
import math

import numpy as np
import torch

from paged_kv_gqa_table_amd import inputs


def _check_tables(case):
    bs = case.block_size
    seen = set()
    for b, n in enumerate(case.seq_lens.tolist()):
        nb = -(-n // bs)
        row = case.block_tables[b].tolist()
        assert all(0 <= r < case.num_blocks for r in row[:nb])
        assert all(r == -1 for r in row[nb:])
        for r in row[:nb]:
            assert r not in seen, "page shared between sequences"
            seen.add(r)


def test_tiny_fp32_shapes_and_seed():
    a = inputs.tiny_fp32()
    b = inputs.tiny_fp32()
    assert a.query.shape == (2, 4, 64) and a.query.dtype == torch.float32
    assert a.key_cache.shape == (16, 2, 16, 64)
    assert a.block_tables.shape == (2, 7)
    assert a.seq_lens.tolist() == [37, 100]
    assert math.isclose(a.scale, 1 / 8)
    for x, y in ((a.query, b.query), (a.key_cache, b.key_cache), (a.value_cache, b.value_cache),
                 (a.block_tables, b.block_tables)):
        assert torch.equal(x, y)
    _check_tables(a)
    c = inputs.tiny_fp32(seed=5)
    assert not torch.equal(a.query, c.query)


def test_llama_gqa4_workload():
    c = inputs.llama_gqa4()
    assert c.query.shape == (32, 32, 128) and c.query.dtype == torch.bfloat16
    lens = c.seq_lens.numpy()
    assert lens.min() >= 512 and lens.max() <= 4096
    pages = int(np.sum(-(-lens // 16)))
    assert c.num_blocks == math.ceil(1.1 * pages)
    assert c.block_tables.shape == (32, -(-int(lens.max()) // 16))
    assert c.num_partitions() == -(-int(lens.max()) // 512)
    _check_tables(c)


def test_layout_round_trip_is_exact():
    for dtype in ("f32", "bf16"):
        c = inputs.make_decode([5, 33, 16], 4, 2, 64, dtype=dtype, seed=3)
        x = c.with_layout(inputs.XPACKED)
        xf = inputs.x_pack_factor(dtype)
        assert x.key_cache.shape == (c.num_blocks, 2, 64 // xf, 16, xf)
        assert x.value_cache.shape == (c.num_blocks, 2, 64, 16)
        # element (blk, h, t, d) of the token-major pool lands where the x-packed layout says
        blk, h, t, d = 3, 1, 7, 37
        assert x.key_cache[blk, h, d // xf, t, d % xf] == c.key_cache[blk, h, t, d]
        assert x.value_cache[blk, h, d, t] == c.value_cache[blk, h, t, d]
        back = x.with_layout(inputs.TOKEN_MAJOR)
        assert torch.equal(back.key_cache, c.key_cache) and torch.equal(back.value_cache, c.value_cache)


def test_nan_canaries_only_touch_invalid_slots():
    c = inputs.make_decode([5, 20], 2, 1, 8, dtype="f32", seed=4, num_blocks=6)
    n = inputs.with_nan_canaries(c)
    bt = c.block_tables
    # valid tokens keep their values
    for b, L in enumerate(c.seq_lens.tolist()):
        for t in range(L):
            blk = int(bt[b, t // 16])
            assert torch.equal(n.key_cache[blk, :, t % 16], c.key_cache[blk, :, t % 16])
    assert torch.isnan(n.key_cache[int(bt[0, 0]), :, 5:]).all()
    owned = {int(bt[0, 0]), int(bt[1, 0]), int(bt[1, 1])}
    for blk in range(6):
        if blk not in owned:
            assert torch.isnan(n.value_cache[blk]).all()


def test_permute_pool_keeps_logical_content():
    c = inputs.make_decode([9, 40], 2, 1, 8, dtype="f32", seed=8)
    p = inputs.permute_pool(c, seed=1)
    for b, L in enumerate(c.seq_lens.tolist()):
        for t in range(L):
            a = c.key_cache[int(c.block_tables[b, t // 16]), :, t % 16]
            z = p.key_cache[int(p.block_tables[b, t // 16]), :, t % 16]
            assert torch.equal(a, z)


def test_mla_workload():
    m = inputs.mla_prefill_b8()
    assert m.batch == 8 and m.q_nope.shape[1:] == (16, 512) and m.q_pe.shape[1:] == (16, 64)
    assert m.ckv_cache.shape[1:] == (1, 512) and m.kpe_cache.shape[1:] == (1, 64)
    ql = (m.qo_indptr[1:] - m.qo_indptr[:-1]).numpy()
    kl = (m.kv_indptr[1:] - m.kv_indptr[:-1]).numpy()
    assert ql.min() >= 1 and ql.max() <= 512
    assert ((kl - ql) >= 0).all() and ((kl - ql) <= 4096).all()
    assert m.num_pages == int(m.kv_indptr[-1])
    assert sorted(m.kv_indices.tolist()) == list(range(m.num_pages))
    assert math.isclose(m.sm_scale, 1 / math.sqrt(192))
