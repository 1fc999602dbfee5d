"""paged_decode_static, the decode entry point that allocates nothing (its partials live in
the library's static device scratch), through the C ABI. Its output is checked against the
existing one-launch paged_decode entry point (same kernels, caller-allocated partials and
counters) and the oracle, under the parity tolerances (f32 1e-5 max-abs; bf16
2e-2 + 1e-2 |ref|, LSE 1e-3), on calls in a row where each later one is smaller than the
one before, so the scratch still holds the previous call's partials. Also: the single-pass
and NUM_SPLITS forms, and the refusal, before any launch, of a call whose partials exceed
the scratch.
"""
import numpy as np
import pytest
import torch

import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_parity_gpu import check_lse, check_out, oracle_subset, say, to_dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().to(torch.float64).numpy()


def _static(case, ps, ns=0):
    dev = to_dev(case)
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode_static(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, case.num_kv_heads,
                            case.max_seq_len, out, lse, partition_size=ps, num_splits=ns, layout=case.layout)
    torch.cuda.synchronize()
    return _np(out), _np(lse)


def _one_launch(case, ps, ns=0):
    """The existing paged_decode entry point with its scratch allocated by the caller."""
    dev = to_dev(case)
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    P = ns if ns > 0 else case.num_partitions(ps)
    out = torch.full((S, H, D), float("nan"), dtype=case.query.dtype, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.empty((S, H, P, D), dtype=torch.float32, device="cuda")
    m = torch.empty((S, H, P), dtype=torch.float32, device="cuda")
    l = torch.empty((S, H, P), dtype=torch.float32, device="cuda")
    counters = torch.zeros((S * case.num_kv_heads,), dtype=torch.int32, device="cuda")
    pkv.paged_decode_into(dev["q"], dev["k"], dev["v"], dev["bt"], dev["lens"], case.scale, case.num_kv_heads, ps,
                          ns, case.max_seq_len, out, lse, acc, m, l, counters, layout=case.layout)
    torch.cuda.synchronize()
    return _np(out), _np(lse)


def _check(case, ps, ns, what):
    say(f"no-alloc decode: {what}")
    out, lse = _static(case, ps, ns)
    ref_out, ref_lse = _one_launch(case, ps, ns)
    check_out(out, ref_out, case.dtype, f"{what}: against paged_decode")
    check_lse(lse, ref_lse, case.dtype, f"{what}: lse against paged_decode")
    ref = oracle_subset(case, list(range(case.num_seqs)))
    check_out(out, ref["out"], case.dtype, f"{what}: against the oracle")
    check_lse(lse, ref["lse"], case.dtype, f"{what}: lse against the oracle")
    empty = case.seq_lens.numpy() == 0
    assert np.all(out[empty] == 0.0) and np.all(np.isneginf(lse[empty])), "empty sequences"


def test_static_scratch_calls_in_a_row_shrinking():
    big = inputs.make_decode([700, 1500, 33, 0, 2100, 512, 4000, 1], 16, 4, 128, dtype="bf16", seed=31)
    small = inputs.make_decode([300, 17, 90, 0], 8, 2, 64, dtype="bf16", layout="xpacked", seed=32)
    tiny_f32 = inputs.make_decode([100, 37], 4, 2, 64, dtype="f32", seed=33)
    _check(big, 512, 0, "bf16 G=4 D=128 token-major, 8 partitions")
    _check(small, 64, 0, "bf16 G=4 D=64 x-packed, 5 partitions (smaller than the call before)")
    _check(tiny_f32, 64, 0, "f32 G=2 D=64, 2 partitions (smaller again)")
    _check(big, 512, 3, "NUM_SPLITS = 3 on the first batch")
    _check(small, 1024, 0, "one partition holds every sequence: the single pass")


def test_static_scratch_matrix_core_and_wide():
    wide = inputs.make_decode([9000, 20000, 0, 513], 24, 4, 256, dtype="bf16", layout="xpacked", seed=34)
    g16 = inputs.make_decode([3000, 15, 700], 32, 2, 128, dtype="bf16", seed=35)
    _check(wide, 512, 0, "bf16 G=6 D=256 x-packed, 40 partitions")
    _check(g16, 512, 0, "bf16 G=16 D=128 (matrix cores), 6 partitions (smaller)")


def test_static_scratch_refuses_what_does_not_fit():
    """256 sequences x 64 heads x 128 partitions x 130 floats (1.09 GB) cannot fit the 64 MiB
    scratch: refused before anything is launched."""
    S, H, KVH, D = 256, 64, 8, 128
    q = torch.zeros((S, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, KVH, 16, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, 4096), dtype=torch.int32, device="cuda")
    lens = torch.zeros((S,), dtype=torch.int32, device="cuda")
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError, match="static scratch"):
        pkv.paged_decode_static(q, k, k, bt, lens, 0.1, KVH, 65536, out)
