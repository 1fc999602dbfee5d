"""GPU parity: the HIP decode path through the C ABI against the float64 oracle.

Tolerances (written here, used everywhere below):
  fp32 inputs:  max |gpu - ref| <= 1e-5 on out, lse, m and acc / l; l relative 1e-5.
  bf16 inputs:  |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise on out and acc / l,
                |lse - ref| <= 1e-3, |m - ref| <= 1e-3, l relative 1e-2.
Full-size workloads are launched exactly as bench.py launches them and every sequence is
compared with the oracle: out, lse and the partials (m, l, acc / l) of every non-empty
partition, exact sentinels past each sequence's last one. The oracle runs one sequence
at a time (the pool is shared), so memory stays bounded at any batch size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_ABS, BF16_REL = 2e-2, 1e-2
LSE_TOL_BF16 = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(case):
    d = "cuda"
    return dict(q=case.query.to(d), k=case.key_cache.to(d), v=case.value_cache.to(d),
                bt=case.block_tables.to(d), lens=case.seq_lens.to(d))


def run_gpu(case, dev=None, partition_size=None, P=None, partials_f64=True):
    """Both phases through the C ABI; returns CPU numpy arrays (float64; with
    partials_f64=False the partial arrays stay float32, for batches whose partials are
    large)."""
    dev = dev or to_dev(case)
    ps = partition_size or case.partition_size
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    P = P or case.num_partitions(ps)
    acc = torch.full((S, H, P, D), float("nan"), dtype=torch.float32, device="cuda")
    m = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((S, H, P), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode_partial(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale,
                             case.num_kv_heads, ps, case.max_seq_len, acc, m, l, layout=case.layout)
    pkv.paged_decode_reduce(acc, m, l, dev["lens"], ps, out, lse)
    torch.cuda.synchronize()
    f = lambda t: t.cpu().to(torch.float64).numpy()
    fp = f if partials_f64 else (lambda t: t.cpu().numpy())
    return dict(out=f(out), lse=f(lse), acc=fp(acc), m=fp(m), l=fp(l), P=P, ps=ps)


def oracle_subset(case, seqs, partition_size=None, P=None, partials=False):
    idx = torch.as_tensor(seqs, dtype=torch.long)
    q = case.query[idx]
    bt = case.block_tables[idx]
    lens = case.seq_lens[idx]
    out, lse = oracle.decode(q, case.key_cache, case.value_cache, case.layout, bt, lens, case.scale,
                             case.num_kv_heads, case.block_size)
    res = dict(out=out, lse=lse)
    if partials:
        ps = partition_size or case.partition_size
        P = P or case.num_partitions(ps)
        acc, m, l = oracle.decode_partials(q, case.key_cache, case.value_cache, case.layout, bt, lens,
                                           case.scale, case.num_kv_heads, case.block_size, ps, P)
        res.update(acc=acc, m=m, l=l)
    return res


def check_out(gpu, ref, dtype, what):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    if dtype == "f32":
        assert err.max(initial=0) <= F32_TOL, f"{what}: max abs err {err.max()}"
    else:
        bound = BF16_ABS + BF16_REL * np.abs(ref)
        bad = err > bound
        rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
        assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max abs {err.max()}, rel {rel}"
    return float(err.max(initial=0))


def check_lse(gpu, ref, dtype, what):
    both_inf = np.isneginf(gpu) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both are -inf: masked out here
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    tol = F32_TOL if dtype == "f32" else LSE_TOL_BF16
    assert np.all(np.isfinite(err)) and err.max(initial=0) <= tol, f"{what}: lse err {err.max()}"


def check_partials(g, r, seqs, lens, ps, dtype, what):
    """m, l and acc / l of every non-empty partition; exact sentinels past P_b."""
    mtol = F32_TOL if dtype == "f32" else 1e-3
    ltol = F32_TOL if dtype == "f32" else 1e-2
    for i, b in enumerate(seqs):
        nb = -(-int(lens[b]) // ps)
        gm, gl, ga = g["m"][b, :, :nb], g["l"][b, :, :nb], g["acc"][b, :, :nb]
        rm, rl, ra = r["m"][i, :, :nb], r["l"][i, :, :nb], r["acc"][i, :, :nb]
        assert np.abs(gm - rm).max(initial=0) <= mtol, f"{what}: m err {np.abs(gm - rm).max()}"
        assert (np.abs(gl - rl) / rl).max(initial=0) <= ltol, f"{what}: l rel err"
        check_out(ga / gl[..., None], ra / rl[..., None], dtype, f"{what}: acc/l")
        # sentinel partitions: m = -inf, l = 0 exactly (up to the grid's partition count)
        P_grid = g["m"].shape[2]
        assert np.all(np.isneginf(g["m"][b, :, nb:P_grid])), f"{what}: sentinel m"
        assert np.all(g["l"][b, :, nb:P_grid] == 0.0), f"{what}: sentinel l"


# --------------------------------------------------------------------------------------
# The workloads
# --------------------------------------------------------------------------------------

def test_tiny_fp32_one_and_two_partitions():
    case = inputs.tiny_fp32()
    say("tiny_fp32: ps=128 (1 partition) and ps=64 (2 partitions)")
    ref = oracle_subset(case, [0, 1], partition_size=64, P=2, partials=True)
    g1 = run_gpu(case, partition_size=128)
    g2 = run_gpu(case, partition_size=64)
    assert g1["P"] == 1 and g2["P"] == 2
    check_out(g1["out"], ref["out"], "f32", "ps=128 out")
    check_out(g2["out"], ref["out"], "f32", "ps=64 out")
    check_lse(g1["lse"], ref["lse"], "f32", "ps=128")
    check_lse(g2["lse"], ref["lse"], "f32", "ps=64")
    assert np.abs(g1["out"] - g2["out"]).max() <= F32_TOL, "1- and 2-partition runs disagree"
    check_partials(g2, ref, [0, 1], case.seq_lens.numpy(), 64, "f32", "tiny partials")
    # seq 0 (37 tokens) has one real partition; partition 1 is its sentinel
    assert np.all(np.isneginf(g2["m"][0, :, 1])) and np.all(g2["l"][0, :, 1] == 0)


def test_llama_gqa4_full():
    case = inputs.llama_gqa4()
    say(f"llama_gqa4: S={case.num_seqs} H={case.num_heads} KVH={case.num_kv_heads} D={case.head_dim}")
    g = run_gpu(case)
    seqs = list(range(case.num_seqs))
    ref = oracle_subset(case, seqs, partials=True)
    err = check_out(g["out"], ref["out"], "bf16", "llama_gqa4 out")
    check_lse(g["lse"], ref["lse"], "bf16", "llama_gqa4")
    check_partials(g, ref, seqs, case.seq_lens.numpy(), 512, "bf16", "llama_gqa4")
    say(f"  max abs err {err:.3e}")


def check_every_sequence(case, results, dtype, what, ps=None):
    """Each sequence of the batch against the oracle, one at a time: out and lse of every
    result in `results` (name -> run_gpu dict over the same batch and partition size),
    and their partials (m, l, acc / l of every non-empty partition, exact sentinels after
    it)."""
    ps = ps or case.partition_size
    lens = case.seq_lens.numpy()
    P = next(iter(results.values()))["P"]
    for b in range(case.num_seqs):
        r = oracle_subset(case, [b], partition_size=ps, P=P, partials=True)
        for name, g in results.items():
            check_out(g["out"][b:b + 1], r["out"], dtype, f"{what} {name} b={b} out")
            check_lse(g["lse"][b:b + 1], r["lse"], dtype, f"{what} {name} b={b}")
            gb = {k: g[k][b:b + 1] for k in ("acc", "m", "l")}
            check_partials(gb, r, [0], lens[b:b + 1], ps, dtype, f"{what} {name} b={b}")
        if b % 8 == 7 or b == case.num_seqs - 1:
            say(f"  {what}: sequences 0..{b} match the oracle (len {int(lens[b])})")


@pytest.mark.timeout(900)
def test_wide_gqa6_both_layouts():
    """Both layouts of the wide-head batch, every sequence and partition against the oracle
    (the token-major copy holds the same values, so one oracle run serves both)."""
    case_x = inputs.wide_gqa6(layout=inputs.XPACKED)
    lens = case_x.seq_lens.numpy()
    say(f"wide_gqa6 x-packed: lens {lens.min()}..{lens.max()}")
    gx = run_gpu(case_x, partials_f64=False)
    torch.cuda.empty_cache()
    case_t = inputs.wide_gqa6(layout=inputs.TOKEN_MAJOR)
    say("wide_gqa6 token-major copy")
    gt = run_gpu(case_t, partials_f64=False)
    del case_t
    torch.cuda.empty_cache()
    check_every_sequence(case_x, {"x-packed": gx, "token-major": gt}, "bf16", "wide_gqa6")
    same = float(np.mean(gt["out"] == gx["out"]))
    say(f"  layouts bitwise-equal fraction {same:.4f}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("long_first", [True, False])
def test_skewed_gqa8(long_first):
    """The skewed batch (one 65,536-token sequence among 127 short ones), every sequence
    and every partition against the oracle, including the 128 partitions of the long one
    and the sentinels of all the empty partitions after each short one."""
    case = inputs.skewed_gqa8(long_first=long_first)
    lens = case.seq_lens.numpy()
    say(f"skewed_gqa8 long_first={long_first}: long sequence at {int(np.argmax(lens))}, {int(lens.max())} tokens")
    g = run_gpu(case, partials_f64=False)
    torch.cuda.empty_cache()
    check_every_sequence(case, {"token-major": g}, "bf16", f"skewed_gqa8 long_first={long_first}")


# --------------------------------------------------------------------------------------
# Edge cases and invariants
# --------------------------------------------------------------------------------------

EDGE_LENS = [0, 1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500]


@pytest.mark.parametrize("dtype,D,H,KVH,layout", [
    ("bf16", 128, 4, 4, "token_major"),   # G=1
    ("bf16", 128, 6, 3, "xpacked"),       # G=2
    ("bf16", 64, 9, 3, "token_major"),    # G=3
    ("bf16", 256, 10, 2, "token_major"),  # G=5
    ("bf16", 256, 14, 2, "xpacked"),      # G=7
    ("bf16", 64, 8, 1, "xpacked"),        # G=8, MQA (matrix cores from here on)
    ("bf16", 128, 16, 2, "xpacked"),      # G=8
    ("bf16", 128, 16, 2, "token_major"),  # G=8
    ("bf16", 128, 32, 2, "token_major"),  # G=16
    ("bf16", 128, 24, 2, "xpacked"),      # G=12
    ("bf16", 256, 20, 2, "token_major"),  # G=10
    ("bf16", 256, 48, 4, "xpacked"),      # G=12
    ("bf16", 64, 6, 1, "token_major"),    # G=6
    ("f32", 64, 4, 4, "xpacked"),
    ("f32", 128, 12, 2, "token_major"),   # G=6
    ("f32", 128, 8, 1, "xpacked"),        # G=8
    ("f32", 256, 4, 2, "token_major"),    # head dim 256
    ("f32", 256, 8, 1, "xpacked"),        # head dim 256, G=8
    ("f32", 64, 24, 2, "token_major"),    # G=12
    ("f32", 128, 16, 1, "xpacked"),       # G=16
    ("f32", 256, 32, 2, "token_major"),   # head dim 256, G=16
    ("f32", 256, 30, 3, "xpacked"),       # head dim 256, G=10
])
def test_edge_lengths(dtype, D, H, KVH, layout):
    say(f"edge: {dtype} D={D} H={H} KVH={KVH} {layout}")
    case = inputs.make_decode(EDGE_LENS, H, KVH, D, dtype=dtype, layout=layout, seed=D + H,
                              partition_size=512)
    seqs = list(range(case.num_seqs))
    for ps in (512, 16, 48):
        g = run_gpu(case, partition_size=ps)
        ref = oracle_subset(case, seqs, partition_size=ps, partials=True)
        check_out(g["out"], ref["out"], dtype, f"ps={ps} out")
        check_lse(g["lse"], ref["lse"], dtype, f"ps={ps}")
        check_partials(g, ref, seqs, case.seq_lens.numpy(), ps, dtype, f"ps={ps}")
        assert np.all(g["out"][0] == 0.0) and np.all(np.isneginf(g["lse"][0])), "empty sequence"


@pytest.mark.parametrize("layout", ["token_major", "xpacked"])
def test_nan_canaries_and_permutation(layout):
    say(f"canaries/permutation {layout}")
    case = inputs.make_decode([700, 33, 1025, 16, 250], 12, 2, 128, dtype="bf16", layout=layout, seed=42,
                              slack=0.5)
    clean = run_gpu(case)
    canary = run_gpu(inputs.with_nan_canaries(case))
    assert np.array_equal(clean["out"], canary["out"]), "canary slots leaked into the output"
    assert np.array_equal(clean["lse"], canary["lse"])
    perm = run_gpu(inputs.permute_pool(case, seed=3))
    assert np.array_equal(clean["out"], perm["out"]), "page permutation changed the result"
    again = run_gpu(case)
    assert np.array_equal(clean["out"], again["out"]) and np.array_equal(clean["m"], again["m"]), \
        "not deterministic"
    ref = oracle_subset(case, list(range(case.num_seqs)))
    check_out(clean["out"], ref["out"], "bf16", "canary case out")


@pytest.mark.parametrize("S,dtype,D,H,KVH,layout", [
    (300, "bf16", 128, 16, 4, "token_major"),   # > 128 sequences: partial items in sequence order
    (300, "bf16", 128, 32, 2, "xpacked"),       # same, matrix-core kernel (G=16)
    (300, "f32", 64, 8, 2, "token_major"),
    (4100, "bf16", 64, 8, 2, "token_major"),    # > 4096 sequences: plain partition grid
    (4100, "bf16", 128, 24, 2, "xpacked"),      # same, matrix-core kernel (G=12)
])
def test_many_sequences(S, dtype, D, H, KVH, layout):
    say(f"many sequences: S={S} {dtype} D={D} H={H} KVH={KVH} {layout}")
    rng = np.random.default_rng(S + D + H)
    lens = rng.integers(0, 200, S)
    lens[::7] = 0
    lens[1::11] = 128   # whole partitions only
    lens[2::13] = 64
    case = inputs.make_decode(lens, H, KVH, D, dtype=dtype, layout=layout, seed=S + H, partition_size=64)
    ps = 64
    g = run_gpu(case, partition_size=ps)
    seqs = list(range(S))
    ref = oracle_subset(case, seqs, partition_size=ps, partials=True)
    check_out(g["out"][seqs], ref["out"], dtype, "out")
    check_lse(g["lse"][seqs], ref["lse"], dtype, "lse")
    check_partials(g, ref, seqs, lens, ps, dtype, "partials")
    for b in range(S):  # every sequence: finite partials where they exist, sentinels after
        nb = -(-int(lens[b]) // ps)
        assert np.all(np.isneginf(g["m"][b, :, nb:])) and np.all(g["l"][b, :, nb:] == 0), f"sentinel b={b}"
        assert np.all(np.isfinite(g["m"][b, :, :nb])) and np.all(g["l"][b, :, :nb] >= 1.0 - 1e-6), f"b={b}"
        if nb == 0:
            assert np.all(g["out"][b] == 0.0) and np.all(np.isneginf(g["lse"][b])), f"empty b={b}"


def test_read_bandwidth_helper():
    """The streaming-read measurement helper runs on odd sizes and leaves the sink alone
    (the fold of a buffer of ones never equals the kernel's marker value)."""
    for n in (4, 4 * 1000 + 4, 1 << 22):
        buf = torch.ones(n, dtype=torch.int32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"read_bandwidth: {n * 4} bytes")
        pkv.read_bandwidth(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0
