"""Cache options in every decode mode, through the C ABI (paged_decode_partial_ex and
paged_decode_ex, reached through the binding's cache options), against the float64 oracle:
float8 e4m3 K/V caches with k_scale / v_scale and ALiBi slopes, in both cache layouts, on
the vector-ALU kernels (G <= 8, bf16 and f32) and the matrix-core kernel (G = 8..16), each in
the four modes: fixed partitions (partials + reduce), NUM_SPLITS (partials + reduce), the
one-launch decode, and the single pass.

Tolerances: those of test_parity_gpu.py (bf16 2e-2 + 1e-2 |ref| on out and acc / l, LSE
1e-3, m 1e-3, l relative 1e-2; f32 1e-5), except the f32 partial max m under ALiBi: its
bias is up to slope * len (hundreds), and float32 holds a number of that size only to a
relative 2^-24 (a spacing of 6e-5 at 1000), so the bound there is 1e-5 + 8 u |m| with
u = 2^-24: the stored m passes through about seven roundings of that relative size (slope
times log2 e, the bias product and sums, and the conversion back by ln 2). The kernels keep
the bias partition-relative and add the constant part to the stored max only, so l, acc / l,
the output and the LSE keep their plain bounds.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_parity_gpu import F32_TOL, check_lse, check_out, say

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500]
U32 = 2.0 ** -24

CASES = [  # (dtype, D, H, KVH, layout)
    ("bf16", 128, 8, 2, "token_major"),   # G=4, vector ALU
    ("bf16", 256, 12, 2, "xpacked"),      # G=6, vector ALU
    ("bf16", 64, 3, 3, "token_major"),    # G=1
    ("bf16", 128, 16, 2, "token_major"),  # G=8, matrix cores
    ("bf16", 128, 24, 2, "xpacked"),      # G=12, matrix cores
    ("bf16", 256, 32, 2, "token_major"),  # G=16, matrix cores
    ("bf16", 64, 16, 1, "xpacked"),       # G=16, D=64, matrix cores
]
OPTIONS = [("fp8", False), ("fp8", True), ("auto", True)]  # (kv_cache_dtype, alibi)


def _np(t):
    return t.cpu().to(torch.float64).numpy()


def _slopes(H):
    """The geometric ALiBi slopes for H heads (Press, Smith and Lewis): 2^(-8 (h + 1) / H)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def _check_partials(acc, m, l, ref, lens, ranges_of, dtype, what):
    racc, rm, rl = ref
    for b, n in enumerate(lens):
        nb = len(ranges_of(int(n)))
        gm, gl, ga = m[b, :, :nb], l[b, :, :nb], acc[b, :, :nb]
        em, el, ea = rm[b, :, :nb], rl[b, :, :nb], racc[b, :, :nb]
        if dtype == "f32":
            mtol = F32_TOL + 8 * U32 * np.abs(em)
            ltol = F32_TOL
        else:
            mtol, ltol = 1e-3, 1e-2
        assert np.all(np.abs(gm - em) <= mtol), f"{what}: m err {np.abs(gm - em).max()} b={b}"
        assert (np.abs(gl - el) / el).max(initial=0) <= ltol, f"{what}: l rel err b={b}"
        check_out(ga / gl[..., None], ea / el[..., None], dtype, f"{what}: acc/l b={b}")
        assert np.all(np.isneginf(m[b, :, nb:])) and np.all(l[b, :, nb:] == 0.0), f"{what}: sentinels b={b}"


def _run_modes(case, kpool, vpool, kv_dtype, slopes, k_scale, v_scale, tag):
    """The four decode modes on one case; every result against the oracle."""
    dev = "cuda"
    q, bt, lens_d = case.query.to(dev), case.block_tables.to(dev), case.seq_lens.to(dev)
    kc, vc = kpool.to(dev), vpool.to(dev)
    S, H, D, KVH = case.num_seqs, case.num_heads, case.head_dim, case.num_kv_heads
    dt = case.dtype
    opts = dict(kv_cache_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                alibi_slopes=None if slopes is None else slopes.to(dev))
    ora = dict(alibi_slopes=slopes, k_scale=k_scale, v_scale=v_scale)
    lens = case.seq_lens.numpy()
    ref_out, ref_lse = oracle.decode(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                                     case.scale, KVH, case.block_size, **ora)

    def bufs(P):
        return (torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, P), float("nan"), dtype=torch.float32, device=dev),
                torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device=dev),
                torch.full((S, H), float("nan"), dtype=torch.float32, device=dev))

    # fixed partitions, two phases
    ps = 512
    P = case.num_partitions(ps)
    say(f"{tag}: fixed partitions ps={ps}")
    acc, m, l, out, lse = bufs(P)
    pkv.paged_decode_partial(q, kc, vc, bt, lens_d, case.scale, KVH, ps, case.max_seq_len, acc, m, l,
                             layout=case.layout, **opts)
    pkv.paged_decode_reduce(acc, m, l, lens_d, ps, out, lse)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                               case.scale, KVH, case.block_size, ps, P, **ora)
    _check_partials(_np(acc), _np(m), _np(l), r, lens, lambda n: oracle.partition_ranges(n, 16, ps), dt,
                    f"{tag} ps={ps}")
    check_out(_np(out), ref_out, dt, f"{tag} ps={ps} out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} ps={ps}")

    # NUM_SPLITS, two phases
    ns = 3
    say(f"{tag}: NUM_SPLITS={ns}")
    acc, m, l, out, lse = bufs(ns)
    pkv.paged_decode_split_partial(q, kc, vc, bt, lens_d, case.scale, KVH, case.max_seq_len, acc, m, l,
                                   layout=case.layout, **opts)
    pkv.paged_decode_split_reduce(acc, m, l, lens_d, case.block_size, out, lse)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, kpool, vpool, case.layout, case.block_tables, case.seq_lens,
                               case.scale, KVH, case.block_size, 0, ns, num_splits=ns, **ora)
    _check_partials(_np(acc), _np(m), _np(l), r, lens, lambda n: oracle.partition_ranges(n, 16, 0, ns), dt,
                    f"{tag} NS={ns}")
    check_out(_np(out), ref_out, dt, f"{tag} NS={ns} out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} NS={ns}")

    # one launch (48-token partitions, combined by the last workgroup), twice on one counter set
    ps = 48
    P = case.num_partitions(ps)
    counters = torch.zeros((S * KVH,), dtype=torch.int32, device=dev)
    for rep in range(2):
        say(f"{tag}: one launch ps={ps} rep={rep}")
        acc, m, l, out, lse = bufs(P)
        pkv.paged_decode_into(q, kc, vc, bt, lens_d, case.scale, KVH, ps, 0, case.max_seq_len, out, lse, acc, m,
                              l, counters, layout=case.layout, **opts)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0, "counters not reset"
        check_out(_np(out), ref_out, dt, f"{tag} one launch out")
        check_lse(_np(lse), ref_lse, dt, f"{tag} one launch")

    # single pass
    say(f"{tag}: single pass")
    _, _, _, out, lse = bufs(1)
    pkv.paged_decode_into(q, kc, vc, bt, lens_d, case.scale, KVH, 512, 0, case.max_seq_len, out, lse,
                          layout=case.layout, **opts)
    torch.cuda.synchronize()
    check_out(_np(out), ref_out, dt, f"{tag} single pass out")
    check_lse(_np(lse), ref_lse, dt, f"{tag} single pass")


@pytest.mark.parametrize("kv_dtype,alibi", OPTIONS)
@pytest.mark.parametrize("dtype,D,H,KVH,layout", CASES)
def test_cache_options_every_mode(dtype, D, H, KVH, layout, kv_dtype, alibi):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout=layout, seed=31 * D + H)
    if kv_dtype == "fp8":
        kpool, vpool = inputs.fp8_pools(case, layout)
        k_scale, v_scale = 0.5, 2.0
    else:
        kpool, vpool = case.key_cache, case.value_cache
        k_scale = v_scale = 1.0
    slopes = _slopes(H) if alibi else None
    tag = f"{dtype} D={D} G={H // KVH} {layout} {kv_dtype} alibi={alibi}"
    _run_modes(case, kpool, vpool, kv_dtype, slopes, k_scale, v_scale, tag)


@pytest.mark.parametrize("D,H,KVH,layout", [(64, 6, 2, "token_major"), (128, 8, 1, "xpacked"),
                                            (128, 4, 4, "token_major"), (256, 16, 1, "xpacked")])
def test_f32_alibi_real_slopes_every_mode(D, H, KVH, layout):
    """f32 with the usual geometric ALiBi slopes (maxima of several hundred at 1500 tokens),
    all four modes, under the f32 bounds (m relative, see the module docstring)."""
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype="f32", layout=layout, seed=37 * D + H)
    _run_modes(case, case.key_cache, case.value_cache, "auto", _slopes(H), 1.0, 1.0,
               f"f32 D={D} G={H // KVH} {layout} alibi")
