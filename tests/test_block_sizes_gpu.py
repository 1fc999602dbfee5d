"""Pools of block sizes other than 16 (the generic-block-size kernel), through the C ABI,
against the float64 oracle, in every decode mode: fixed partitions (partials + reduce),
NUM_SPLITS (partials + reduce), the one-launch decode and the single pass; with float8
caches and ALiBi; and the PagedAttention V2 entry point at block sizes 8 and 32.

Tolerances are those of test_parity_gpu.py (bf16 2e-2 + 1e-2 |ref| on out and acc / l,
LSE 1e-3, m 1e-3, l relative 1e-2; f32 1e-5, with the f32 partial max under ALiBi bounded
by 1e-5 + 8 u |m| as in test_cache_options_gpu.py).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_cache_options_gpu import _check_partials, _np, _slopes
from tests.test_parity_gpu import check_lse, check_out, say

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 7, 8, 9, 31, 32, 33, 100, 511, 512, 513, 1500]

CASES = [  # (dtype, D, H, KVH, layout, block_size)
    ("bf16", 128, 8, 2, "token_major", 8),    # G=4
    ("bf16", 256, 12, 2, "xpacked", 32),      # G=6
    ("bf16", 64, 16, 1, "xpacked", 8),        # G=16
    ("bf16", 128, 24, 2, "token_major", 32),  # G=12
    ("bf16", 128, 4, 4, "token_major", 64),   # G=1
    ("bf16", 64, 6, 2, "xpacked", 1),         # one token per block
    ("f32", 128, 6, 2, "token_major", 32),    # G=3
    ("f32", 64, 16, 2, "xpacked", 8),         # G=8
    ("f32", 256, 4, 1, "xpacked", 32),        # G=4, head dim 256
    ("bf16", 64, 24, 2, "token_major", 16),   # G=12 at head dim 64 token-major: the generic kernel too
]


def _run_modes(case, kpool, vpool, kv_dtype, slopes, k_scale, v_scale, tag):
    dev = "cuda"
    q, bt, lens_d = case.query.to(dev), case.block_tables.to(dev), case.seq_lens.to(dev)
    kc, vc = kpool.to(dev), vpool.to(dev)
    S, H, D, KVH, bs = case.num_seqs, case.num_heads, case.head_dim, case.num_kv_heads, case.block_size
    dt = case.dtype
    opts = dict(kv_cache_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                alibi_slopes=None if slopes is None else slopes.to(dev))
    ora = dict(alibi_slopes=slopes, k_scale=k_scale, v_scale=v_scale)
    lens = case.seq_lens.numpy()
    ref_out, ref_lse = oracle.decode(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                                     case.scale, KVH, bs, **ora)

    def bufs(P):
        return (torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device=dev),
                torch.full((S, H), float("nan"), dtype=torch.float32, device=dev))

    ps = max(bs, 64) * 4  # a multiple of the block size, several partitions at 1500 tokens
    P = -(-case.max_seq_len // ps)
    say(f"{tag}: fixed partitions ps={ps}")
    acc, m, l, out, lse = bufs(P)
    pkv.paged_decode_partial(q, kc, vc, bt, lens_d, case.scale, KVH, ps, case.max_seq_len, acc, m, l,
                             layout=case.layout, **opts)
    pkv.paged_decode_reduce(acc, m, l, lens_d, ps, out, lse)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                               case.scale, KVH, bs, ps, P, **ora)
    _check_partials(_np(acc), _np(m), _np(l), r, lens, lambda n: oracle.partition_ranges(n, bs, ps), dt,
                    f"{tag} ps={ps}")
    check_out(_np(out), ref_out, dt, f"{tag} ps={ps} out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} ps={ps}")

    ns = 3
    say(f"{tag}: NUM_SPLITS={ns}")
    acc, m, l, out, lse = bufs(ns)
    pkv.paged_decode_split_partial(q, kc, vc, bt, lens_d, case.scale, KVH, case.max_seq_len, acc, m, l,
                                   layout=case.layout, **opts)
    pkv.paged_decode_split_reduce(acc, m, l, lens_d, bs, out, lse)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                               case.scale, KVH, bs, 0, ns, num_splits=ns, **ora)
    _check_partials(_np(acc), _np(m), _np(l), r, lens, lambda n: oracle.partition_ranges(n, bs, 0, ns), dt,
                    f"{tag} NS={ns}")
    check_out(_np(out), ref_out, dt, f"{tag} NS={ns} out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} NS={ns}")

    ps1 = max(bs, 32) * 3  # one launch: short partitions, combined by the last workgroup
    P1 = -(-case.max_seq_len // ps1)
    counters = torch.zeros((S * KVH,), dtype=torch.int32, device=dev)
    for rep in range(2):
        say(f"{tag}: one launch ps={ps1} rep={rep}")
        acc, m, l, out, lse = bufs(P1)
        pkv.paged_decode_into(q, kc, vc, bt, lens_d, case.scale, KVH, ps1, 0, case.max_seq_len, out, lse, acc, m,
                              l, counters, layout=case.layout, **opts)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0, "counters not reset"
        check_out(_np(out), ref_out, dt, f"{tag} one launch out")
        check_lse(_np(lse), ref_lse, dt, f"{tag} one launch")

    say(f"{tag}: single pass")
    _, _, _, out, lse = bufs(1)
    pkv.paged_decode_into(q, kc, vc, bt, lens_d, case.scale, KVH, ps, 0, case.max_seq_len, out, lse,
                          layout=case.layout, **opts)
    torch.cuda.synchronize()
    check_out(_np(out), ref_out, dt, f"{tag} single pass out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} single pass")


@pytest.mark.parametrize("dtype,D,H,KVH,layout,bs", CASES)
def test_block_size_every_mode(dtype, D, H, KVH, layout, bs):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout=layout, block_size=bs, seed=7 * D + H + bs)
    _run_modes(case, case.key_cache, case.value_cache, "auto", None, 1.0, 1.0,
               f"{dtype} D={D} G={H // KVH} {layout} bs={bs}")


@pytest.mark.parametrize("D,H,KVH,layout,bs", [(128, 8, 2, "token_major", 32), (64, 16, 1, "xpacked", 8)])
def test_block_size_fp8_alibi(D, H, KVH, layout, bs):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype="bf16", layout=layout, block_size=bs, seed=11 * D + bs)
    kpool, vpool = inputs.fp8_pools(case, layout)
    _run_modes(case, kpool, vpool, "fp8", _slopes(H), 0.5, 2.0, f"fp8+alibi D={D} G={H // KVH} {layout} bs={bs}")


@pytest.mark.parametrize("dtype,bs", [("bf16", 8), ("bf16", 32), ("f32", 32)])
def test_paged_attention_v2_block_sizes(dtype, bs):
    """The PagedAttention V2 entry point (x-packed cache, 512-token partitions) at block
    sizes 8 and 32: normalized partials, exp_sums, max_logits and the output."""
    D, H, KVH = 128, 8, 2
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout="xpacked", block_size=bs, seed=13 + bs)
    dev = "cuda"
    S = case.num_seqs
    P = -(-case.max_seq_len // 512)
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device=dev)
    ml = torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev)
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev)
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device=dev)
    say(f"paged_attention_v2 {dtype} bs={bs}")
    pkv.paged_attention_v2(out, es, ml, tmp, case.query.to(dev), case.key_cache.to(dev), case.value_cache.to(dev),
                           KVH, case.scale, case.block_tables.to(dev), case.seq_lens.to(dev), bs, case.max_seq_len)
    torch.cuda.synchronize()
    ref_out, _ = oracle.decode(case.query, case.key_cache, case.value_cache, "xpacked", case.block_tables,
                               case.seq_lens, case.scale, KVH, bs)
    check_out(_np(out), ref_out, dtype, "v2 out")
    racc, rm, rl = oracle.decode_partials(case.query, case.key_cache, case.value_cache, "xpacked", case.block_tables,
                                          case.seq_lens, case.scale, KVH, bs, 512, P)
    lens = case.seq_lens.numpy()
    for b, n in enumerate(lens):
        nb = len(oracle.partition_ranges(int(n), bs, 512))
        check_out(_np(tmp)[b, :, :nb], racc[b, :, :nb] / rl[b, :, :nb, None], dtype, f"v2 tmp_output b={b}")
        assert np.all(np.abs(_np(ml)[b, :, :nb] - rm[b, :, :nb]) <= (1e-3 if dtype == "bf16" else 1e-5))
        assert np.all(np.abs(_np(es)[b, :, :nb] / rl[b, :, :nb] - 1) <= (1e-2 if dtype == "bf16" else 1e-5))
