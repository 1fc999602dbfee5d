"""GPU parity of the decode entry points beyond the two fixed-partition phases, through the
C ABI, against the float64 oracle:
  * paged_decode: the whole decode in one launch (single pass with one partition per
    sequence; otherwise the last workgroup of each (sequence, kv head) combines);
  * paged_decode_split_partial / _split_reduce: NUM_SPLITS page-aligned splits;
  * paged_attention_v2: normalized partials (tmp_output, exp_sums, max_logits).
Tolerances are those of test_parity_gpu.py (f32 1e-5 max-abs; bf16 2e-2 + 1e-2 |ref|,
LSE 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_parity_gpu import (F32_TOL, check_lse, check_out, oracle_subset, run_gpu, say,
                                   to_dev)

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500]

# (dtype, D, H, KVH, layout): every kernel family (vector-ALU bf16 and f32, matrix cores)
CONFIGS = [
    ("bf16", 128, 8, 2, "token_major"),   # G=4, vector ALU
    ("bf16", 256, 12, 2, "xpacked"),      # G=6, vector ALU
    ("bf16", 64, 3, 3, "token_major"),    # G=1
    ("bf16", 128, 16, 2, "token_major"),  # G=8, matrix cores
    ("bf16", 256, 24, 2, "xpacked"),      # G=12, matrix cores
    ("f32", 128, 6, 2, "token_major"),    # G=3, f32
    ("f32", 64, 8, 1, "xpacked"),         # G=8, f32
    ("f32", 256, 12, 1, "xpacked"),       # G=12, f32 head dim 256
]


def _np(t):
    return t.cpu().to(torch.float64).numpy()


def one_launch(case, dev, ps, P, num_splits=0, counters=None, keep_partials=True):
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    acc = m = l = None
    if keep_partials:
        acc = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
        if counters is None:
            counters = torch.zeros(S * case.num_kv_heads, dtype=torch.int32, device="cuda")
    pkv.paged_decode_into(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, case.num_kv_heads,
                          ps, num_splits, case.max_seq_len, out, lse, acc, m, l, counters, layout=case.layout)
    torch.cuda.synchronize()
    return _np(out), _np(lse), counters


@pytest.mark.parametrize("dtype,D,H,KVH,layout", CONFIGS)
def test_one_launch_fixed_partitions(dtype, D, H, KVH, layout):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout=layout, seed=7 * D + H)
    dev = to_dev(case)
    ref = oracle_subset(case, list(range(case.num_seqs)))
    counters = torch.zeros(case.num_seqs * KVH, dtype=torch.int32, device="cuda")
    for ps in (512, 16, 48):
        P = case.num_partitions(ps)
        say(f"one launch: {dtype} D={D} H={H} KVH={KVH} {layout} ps={ps} P={P}")
        for rep in range(2):  # the same counters twice: the first call must leave them zero
            out, lse, counters = one_launch(case, dev, ps, P, counters=counters)
            assert int(counters.abs().sum().item()) == 0, "counters not reset"
            check_out(out, ref["out"], dtype, f"ps={ps} rep={rep} out")
            check_lse(lse, ref["lse"], dtype, f"ps={ps} rep={rep}")
            assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0])), "empty sequence"


@pytest.mark.parametrize("dtype,D,H,KVH,layout", CONFIGS)
def test_single_pass(dtype, D, H, KVH, layout):
    """One partition per sequence whatever its length: no partials, no counters."""
    case = inputs.make_decode(EDGE_LENS + [2100], H, KVH, D, dtype=dtype, layout=layout, seed=3 * D + H)
    say(f"single pass: {dtype} D={D} H={H} KVH={KVH} {layout}")
    out, lse, _ = one_launch(case, to_dev(case), 512, 1, keep_partials=False)
    ref = oracle_subset(case, list(range(case.num_seqs)))
    check_out(out, ref["out"], dtype, "single pass out")
    check_lse(lse, ref["lse"], dtype, "single pass")


def _check_ranged_partials(acc, m, l, r, lens, ranges_of, dtype, what, normalized=False):
    ltol = F32_TOL if dtype == "f32" else 1e-2
    for b, n in enumerate(lens):
        nb = len(ranges_of(int(n)))
        gm, gl, ga = m[b, :, :nb], l[b, :, :nb], acc[b, :, :nb]
        rm, rl, ra = r[1][b, :, :nb], r[2][b, :, :nb], r[0][b, :, :nb]
        # f32: 1e-5 plus 8 float32 rounding units of |m| (an ALiBi max runs into the
        # hundreds, where float32 itself is spaced 3e-5 and more; see test_cache_options_gpu)
        mtol = F32_TOL + 8 * 2.0 ** -24 * np.abs(rm) if dtype == "f32" else 1e-3
        assert np.all(np.abs(gm - rm) <= mtol), f"{what}: m err {np.abs(gm - rm).max()}"
        assert (np.abs(gl - rl) / rl).max(initial=0) <= ltol, f"{what}: l rel err"
        if normalized:
            check_out(ga, ra, dtype, f"{what}: normalized acc b={b}")
        else:
            check_out(ga / gl[..., None], ra / rl[..., None], dtype, f"{what}: acc/l b={b}")
        assert np.all(np.isneginf(m[b, :, nb:])) and np.all(l[b, :, nb:] == 0.0), f"{what}: sentinels b={b}"


@pytest.mark.parametrize("dtype,D,H,KVH,layout", CONFIGS)
def test_split_policy(dtype, D, H, KVH, layout):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout=layout, seed=5 * D + H)
    dev = to_dev(case)
    S = case.num_seqs
    lens = case.seq_lens.numpy()
    ref_out = oracle_subset(case, list(range(S)))
    for ns in (1, 3, 7, 16):
        say(f"NUM_SPLITS={ns}: {dtype} D={D} H={H} KVH={KVH} {layout}")
        acc = torch.full((S, H, ns, D), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
        lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_decode_split_partial(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, KVH,
                                       case.max_seq_len, acc, m, l, layout=layout)
        pkv.paged_decode_split_reduce(acc, m, l, dev["lens"], case.block_size, out, lse)
        torch.cuda.synchronize()
        r = oracle.decode_partials(case.query, case.key_cache, case.value_cache, layout, case.block_tables,
                                   case.seq_lens, case.scale, KVH, case.block_size, 0, ns, num_splits=ns)
        _check_ranged_partials(_np(acc), _np(m), _np(l), r, lens,
                               lambda n: oracle.partition_ranges(n, case.block_size, 0, ns), dtype, f"NS={ns}")
        check_out(_np(out), ref_out["out"], dtype, f"NS={ns} out")
        check_lse(_np(lse), ref_out["lse"], dtype, f"NS={ns}")
        o1, s1, _ = one_launch(case, dev, 0, ns, num_splits=ns)
        check_out(o1, ref_out["out"], dtype, f"NS={ns} one-launch out")
        check_lse(s1, ref_out["lse"], dtype, f"NS={ns} one-launch")


@pytest.mark.parametrize("dtype,D,H,KVH", [("bf16", 128, 8, 2), ("bf16", 256, 24, 4), ("bf16", 128, 16, 2),
                                           ("f32", 64, 4, 2)])
def test_paged_attention_v2(dtype, D, H, KVH):
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout="xpacked", seed=11 * D + H)
    dev = to_dev(case)
    S = case.num_seqs
    P = case.num_partitions(512)
    say(f"paged_attention_v2: {dtype} D={D} H={H} KVH={KVH} P={P}")
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    ml = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    pkv.paged_attention_v2(out, es, ml, tmp, dev["q"], dev["k"], dev["v"], KVH, case.scale, dev["bt"],
                           dev["lens"], case.block_size, case.max_seq_len)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, case.key_cache, case.value_cache, "xpacked", case.block_tables,
                               case.seq_lens, case.scale, KVH, case.block_size, 512, P, normalized=True)
    _check_ranged_partials(_np(tmp), _np(ml), _np(es), r, case.seq_lens.numpy(),
                           lambda n: oracle.partition_ranges(n, case.block_size, 512), dtype, "v2", normalized=True)
    ref = oracle_subset(case, list(range(S)))
    check_out(_np(out), ref["out"], dtype, "v2 out")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("workload", ["llama_gqa4", "wide_gqa6", "skewed_gqa8"])
def test_one_launch_full_size(workload):
    """The benchmarked workloads through the one-launch entry point, in the launch
    configuration the bench times: against the two-phase result and the oracle on every
    sequence."""
    case = inputs.decode_workload(workload)
    say(f"one launch full size: {workload}")
    dev = to_dev(case)
    ps = case.partition_size
    P = case.num_partitions(ps)
    two = run_gpu(case, dev=dev)
    out, lse, counters = one_launch(case, dev, ps, P)
    assert int(counters.abs().sum().item()) == 0
    check_out(out, two["out"], case.dtype, "one launch vs two phases")
    for b in range(case.num_seqs):
        ref = oracle_subset(case, [b])
        check_out(out[b:b + 1], ref["out"], case.dtype, f"one launch out b={b}")
        check_lse(lse[b:b + 1], ref["lse"], case.dtype, f"one launch lse b={b}")


def test_lengths_past_max_seq_len_stay_in_bounds():
    """A length above max_seq_len breaks the contract; the partial arrays of the other
    sequences and the memory after them must still be untouched (lengths are cut to the
    partitions the arrays hold)."""
    case = inputs.make_decode([1000, 300, 200], 8, 2, 128, dtype="bf16", seed=9)
    dev = to_dev(case)
    S, H, D, ps = 3, 8, 128, 512
    P = 1  # max_seq_len = 300 -> one partition; sequence 0 claims 1000 tokens
    guard = 4096
    acc_buf = torch.full((S * H * P * D + guard,), float("nan"), dtype=torch.float32, device="cuda")
    m_buf = torch.full((S * H * P + guard,), float("nan"), dtype=torch.float32, device="cuda")
    l_buf = torch.full((S * H * P + guard,), float("nan"), dtype=torch.float32, device="cuda")
    acc = acc_buf[:S * H * P * D].view(S, H, P, D)
    m = m_buf[:S * H * P].view(S, H, P)
    l = l_buf[:S * H * P].view(S, H, P)
    say("lengths past max_seq_len")
    pkv.paged_decode_partial(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, 2, ps, 300,
                             acc, m, l)
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    pkv.paged_decode_reduce(acc, m, l, dev["lens"], ps, out)
    torch.cuda.synchronize()
    assert torch.isnan(acc_buf[S * H * P * D:]).all() and torch.isnan(m_buf[S * H * P:]).all() \
        and torch.isnan(l_buf[S * H * P:]).all(), "write past the partial arrays"
    ref = oracle_subset(case, [1, 2])
    check_out(_np(out)[1:], ref["out"], "bf16", "sequences within the contract")


@pytest.mark.parametrize("dtype,D,H,KVH", [("bf16", 128, 8, 2), ("bf16", 256, 12, 2), ("bf16", 128, 16, 2),
                                           ("bf16", 128, 32, 2), ("f32", 64, 6, 3)])
def test_paged_attention_v2_alibi(dtype, D, H, KVH):
    """ALiBi slopes through the PagedAttention V2 entry point, several partitions per
    sequence (each score biased by its absolute position)."""
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout="xpacked", seed=13 * D + H)
    dev = to_dev(case)
    S = case.num_seqs
    P = case.num_partitions(512)
    # the usual geometric slopes (f32 maxima then run into the hundreds: relative m bound)
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)
    say(f"paged_attention_v2 + ALiBi: {dtype} D={D} H={H} KVH={KVH}")
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    ml = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    pkv.paged_attention_v2(out, es, ml, tmp, dev["q"], dev["k"], dev["v"], KVH, case.scale, dev["bt"],
                           dev["lens"], case.block_size, case.max_seq_len, alibi_slopes=slopes.to("cuda"))
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, case.key_cache, case.value_cache, "xpacked", case.block_tables,
                               case.seq_lens, case.scale, KVH, case.block_size, 512, P, normalized=True,
                               alibi_slopes=slopes)
    _check_ranged_partials(_np(tmp), _np(ml), _np(es), r, case.seq_lens.numpy(),
                           lambda n: oracle.partition_ranges(n, case.block_size, 512), dtype, "v2 alibi",
                           normalized=True)
    ref, _ = oracle.decode(case.query, case.key_cache, case.value_cache, "xpacked", case.block_tables,
                           case.seq_lens, case.scale, KVH, case.block_size, alibi_slopes=slopes)
    check_out(_np(out), ref, dtype, "v2 alibi out")


@pytest.mark.parametrize("D,H,KVH,alibi", [(128, 8, 2, False), (256, 24, 4, False), (64, 4, 4, False),
                                          (128, 16, 2, True)])
def test_paged_attention_v2_fp8_cache(D, H, KVH, alibi):
    """float8 e4m3 caches (x-packed, x = 16) with k_scale / v_scale through the PagedAttention
    V2 entry point: partials and output against the oracle on the same float8 pools."""
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype="bf16", layout="xpacked", seed=17 * D + H)
    k8, v8 = inputs.fp8_xpacked_pools(case)
    S, P = case.num_seqs, case.num_partitions(512)
    k_scale, v_scale = 0.5, 2.0
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32) if alibi else None
    say(f"paged_attention_v2 fp8 cache: D={D} H={H} KVH={KVH} alibi={alibi}")
    dev = to_dev(case)
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    ml = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_v2(out, es, ml, tmp, dev["q"], k8.to("cuda"), v8.to("cuda"), KVH, case.scale, dev["bt"],
                           dev["lens"], case.block_size, case.max_seq_len,
                           alibi_slopes=None if slopes is None else slopes.to("cuda"), kv_cache_dtype="fp8",
                           k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    r = oracle.decode_partials(case.query, k8, v8, "xpacked", case.block_tables, case.seq_lens, case.scale, KVH,
                               case.block_size, 512, P, normalized=True, alibi_slopes=slopes, k_scale=k_scale,
                               v_scale=v_scale)
    _check_ranged_partials(_np(tmp), _np(ml), _np(es), r, case.seq_lens.numpy(),
                           lambda n: oracle.partition_ranges(n, case.block_size, 512), "bf16", "v2 fp8",
                           normalized=True)
    ref, _ = oracle.decode(case.query, k8, v8, "xpacked", case.block_tables, case.seq_lens, case.scale, KVH,
                           case.block_size, alibi_slopes=slopes, k_scale=k_scale, v_scale=v_scale)
    check_out(_np(out), ref, "bf16", "v2 fp8 out")


def test_python_paged_decode_defaults():
    """The Python wrapper: default (two launches when there are several partitions, one when
    a single partition holds every sequence), NUM_SPLITS, and lse output."""
    case = inputs.make_decode([3, 700, 1500, 0], 8, 2, 128, dtype="bf16", seed=23)
    dev = to_dev(case)
    ref = oracle_subset(case, list(range(case.num_seqs)))
    args = (dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, 2)
    say("python paged_decode defaults")
    for kw in (dict(), dict(max_num_partitions=1), dict(num_splits=4), dict(one_launch=True)):
        out, lse = pkv.paged_decode(*args, return_lse=True, **kw)
        torch.cuda.synchronize()
        check_out(_np(out), ref["out"], "bf16", f"paged_decode {kw}")
        check_lse(_np(lse), ref["lse"], "bf16", f"paged_decode {kw}")


@pytest.mark.timeout(900)
def test_llama_gqa4_fp8_full():
    """The llama_gqa4 batch with a float8 e4m3 cache through the PagedAttention V2 entry point,
    as the bench times it (x-packed, x = 16, unit scales): every sequence's normalized
    partials and output against the oracle on the same float8 pools."""
    case = inputs.llama_gqa4()
    k8, v8 = inputs.fp8_xpacked_pools(case)
    S, H, D, KVH = case.num_seqs, case.num_heads, case.head_dim, case.num_kv_heads
    P = case.num_partitions(512)
    dev = to_dev(case)
    say(f"llama_gqa4 float8 cache, full size: S={S} P={P}")
    tmp = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
    es = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    ml = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_v2(out, es, ml, tmp, dev["q"], k8.to("cuda"), v8.to("cuda"), KVH, case.scale, dev["bt"],
                           dev["lens"], case.block_size, case.max_seq_len, kv_cache_dtype="fp8", k_scale=1.0,
                           v_scale=1.0)
    torch.cuda.synchronize()
    tmp, es, ml, out = _np(tmp), _np(es), _np(ml), _np(out)
    lens = case.seq_lens.numpy()
    for b in range(S):
        idx = torch.tensor([b])
        args = (case.query[idx], k8, v8, "xpacked", case.block_tables[idx], case.seq_lens[idx], case.scale, KVH,
                case.block_size)
        r = oracle.decode_partials(*args, 512, P, normalized=True)
        _check_ranged_partials(tmp[b:b + 1], ml[b:b + 1], es[b:b + 1], r, lens[b:b + 1],
                               lambda n: oracle.partition_ranges(n, case.block_size, 512), "bf16", f"fp8 b={b}",
                               normalized=True)
        ref, _ = oracle.decode(*args)
        check_out(out[b:b + 1], ref, "bf16", f"fp8 out b={b}")
    say("  every sequence matches the oracle")


@pytest.mark.timeout(900)
def test_llama_gqa4_num_splits_full():
    """The llama_gqa4 batch under the NUM_SPLITS policy (8 page-aligned splits per sequence),
    both phases: every sequence's split partials, output and LSE against the oracle."""
    case = inputs.llama_gqa4()
    dev = to_dev(case)
    S, H, D, KVH, ns = case.num_seqs, case.num_heads, case.head_dim, case.num_kv_heads, 8
    say(f"llama_gqa4 NUM_SPLITS={ns}, full size")
    acc = torch.full((S, H, ns, D), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode_split_partial(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, KVH,
                                   case.max_seq_len, acc, m, l, layout=case.layout)
    pkv.paged_decode_split_reduce(acc, m, l, dev["lens"], case.block_size, out, lse)
    torch.cuda.synchronize()
    acc, m, l, out, lse = _np(acc), _np(m), _np(l), _np(out), _np(lse)
    lens = case.seq_lens.numpy()
    for b in range(S):
        idx = torch.tensor([b])
        args = (case.query[idx], case.key_cache, case.value_cache, case.layout, case.block_tables[idx],
                case.seq_lens[idx], case.scale, KVH, case.block_size)
        r = oracle.decode_partials(*args, 0, ns, num_splits=ns)
        _check_ranged_partials(acc[b:b + 1], m[b:b + 1], l[b:b + 1], r, lens[b:b + 1],
                               lambda n: oracle.partition_ranges(n, case.block_size, 0, ns), "bf16",
                               f"NS={ns} b={b}")
        ro, rl = oracle.decode(*args)
        check_out(out[b:b + 1], ro, "bf16", f"NS={ns} out b={b}")
        check_lse(lse[b:b + 1], rl, "bf16", f"NS={ns} b={b}")
    say("  every sequence matches the oracle")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,D,H,KVH,layout", [
    ("bf16", 128, 8, 2, "token_major"),   # G=4, vector ALU
    ("bf16", 128, 24, 2, "xpacked"),      # G=12, matrix cores
    ("f32", 64, 4, 2, "token_major"),     # G=2, f32
])
def test_num_splits_ten_thousand_sequences(dtype, D, H, KVH, layout):
    """10,000 sequences under the NUM_SPLITS policy, both phases and the one-launch decode,
    every sequence against the oracle: past the work list's LDS capacity the plain grid
    of (split, sequence, kv head) workgroups takes over."""
    S, ns = 10000, 4
    rng = np.random.default_rng(S + H)
    lens = rng.integers(0, 300, S)
    lens[::9] = 0
    lens[1::13] = 16 * ns * 3   # splits of whole pages only
    lens[2::17] = 1
    case = inputs.make_decode(lens, H, KVH, D, dtype=dtype, layout=layout, seed=S + D + H)
    dev = to_dev(case)
    say(f"NUM_SPLITS={ns}, S={S}: {dtype} D={D} H={H} KVH={KVH} {layout}")
    acc = torch.full((S, H, ns, D), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((S, H, ns), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode_split_partial(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, KVH,
                                   case.max_seq_len, acc, m, l, layout=layout)
    pkv.paged_decode_split_reduce(acc, m, l, dev["lens"], case.block_size, out, lse)
    torch.cuda.synchronize()
    say("  oracle")
    r = oracle.decode_partials(case.query, case.key_cache, case.value_cache, layout, case.block_tables,
                               case.seq_lens, case.scale, KVH, case.block_size, 0, ns, num_splits=ns)
    _check_ranged_partials(_np(acc), _np(m), _np(l), r, lens,
                           lambda n: oracle.partition_ranges(n, case.block_size, 0, ns), dtype, f"NS={ns}")
    ro, rl = oracle.decode(case.query, case.key_cache, case.value_cache, layout, case.block_tables,
                           case.seq_lens, case.scale, KVH, case.block_size)
    check_out(_np(out), ro, dtype, "two phases out")
    check_lse(_np(lse), rl, dtype, "two phases")
    say("  one launch")
    o1, s1, counters = one_launch(case, dev, 0, ns, num_splits=ns)
    assert int(counters.abs().sum().item()) == 0, "counters not reset"
    check_out(o1, ro, dtype, "one-launch out")
    check_lse(s1, rl, dtype, "one-launch")
