"""K/V pools past 4 GiB, through the C ABI: every decode kernel family forms page addresses
in 64 bits. A small batch's blocks are placed above the 4 GiB byte offset of a pool with
more than 2^32 bytes per cache (only the blocks the batch uses are written); phase 1 and
the combine must give the small-pool result bit for bit, and the oracle's output within
the tolerances of test_parity_gpu.py.
"""
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_parity_gpu import check_lse, check_out, say

pytestmark = pytest.mark.gpu

LENS = [700, 1500, 33, 0]
CASES = [  # (dtype, D, H, KVH, layout, block_size, cache)
    ("bf16", 128, 8, 2, "token_major", 16, "auto"),   # vector ALU, G = 4
    ("bf16", 256, 12, 2, "xpacked", 16, "auto"),      # vector ALU, G = 6, x-packed
    ("bf16", 128, 16, 2, "token_major", 16, "auto"),  # matrix cores, G = 8
    ("f32", 128, 8, 2, "token_major", 16, "auto"),    # float32 vector ALU
    ("bf16", 128, 8, 2, "token_major", 32, "auto"),   # the generic-block-size kernel
    ("bf16", 128, 8, 2, "xpacked", 16, "fp8"),        # float8 e4m3 cache
]


def _np(t):
    return t.cpu().to(torch.float64).numpy()


@pytest.mark.parametrize("dtype,D,H,KVH,layout,bs,cache", CASES)
def test_pool_past_4_gib(dtype, D, H, KVH, layout, bs, cache):
    case = inputs.make_decode(LENS, H, KVH, D, dtype=dtype, layout=layout, block_size=bs, seed=7 * D + H + bs)
    if cache == "fp8":
        kpool, vpool = inputs.fp8_pools(case, layout)
        ks, vs = 0.5, 2.0
    else:
        kpool, vpool = case.key_cache, case.value_cache
        ks = vs = 1.0
    dev = "cuda"
    nb = kpool.shape[0]
    block_bytes = kpool[0].numel() * kpool.element_size()
    shift = (1 << 32) // block_bytes + 16  # every used block starts past 4 GiB
    big_nb = shift + nb + 64
    tag = f"{dtype} D={D} G={H // KVH} {layout} bs={bs} {cache}"
    say(f"pool past 4 GiB: {tag}: {big_nb} blocks of {block_bytes} B")
    q, lens = case.query.to(dev), case.seq_lens.to(dev)
    bt = case.block_tables.to(dev)
    bt_big = torch.where(bt >= 0, bt + shift, bt)
    kc, vc = kpool.to(dev), vpool.to(dev)
    S, D_, P, ps = case.num_seqs, case.head_dim, -(-case.max_seq_len // 512), 512
    opts = dict(layout=layout, kv_cache_dtype=cache, k_scale=ks, v_scale=vs)
    kb = torch.empty((big_nb,) + tuple(kpool.shape[1:]), dtype=kpool.dtype, device=dev)
    vb = torch.empty((big_nb,) + tuple(vpool.shape[1:]), dtype=vpool.dtype, device=dev)
    try:
        rows = torch.arange(nb, device=dev) + shift
        # through byte views: index_copy_ has no float8 kernel
        kb.view(torch.uint8).index_copy_(0, rows, kc.view(torch.uint8))
        vb.view(torch.uint8).index_copy_(0, rows, vc.view(torch.uint8))
        results = []
        for k_, v_, t_ in ((kc, vc, bt), (kb, vb, bt_big)):
            acc = torch.full((S, H, P, D_), float("nan"), dtype=torch.float32, device=dev)
            m = torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev)
            l = torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev)
            out = torch.full((S, H, D_), float("nan"), dtype=case.query.dtype, device=dev)
            lse = torch.full((S, H), float("nan"), dtype=torch.float32, device=dev)
            pkv.paged_decode_partial(q, k_, v_, t_, lens, case.scale, KVH, ps, case.max_seq_len, acc, m, l, **opts)
            pkv.paged_decode_reduce(acc, m, l, lens, ps, out, lse)
            torch.cuda.synchronize()
            results.append((acc, m, l, out, lse))
        for a_, b_, name in zip(results[0], results[1], ("acc", "m", "l", "out", "lse")):
            assert torch.equal(a_.nan_to_num(7.0), b_.nan_to_num(7.0)), f"{tag}: {name} differs on the large pool"
        ref_out, ref_lse = oracle.decode(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                                         case.scale, KVH, bs, k_scale=ks, v_scale=vs)
        check_out(_np(results[1][3]), ref_out, dtype, f"{tag} out")
        check_lse(_np(results[1][4]), ref_lse, dtype, f"{tag} lse")
    finally:
        del kb, vb
        torch.cuda.empty_cache()
