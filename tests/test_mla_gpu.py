"""GPU parity of the MLA causal paged prefill against the float64 oracle.

Tolerances (as for every bf16 output here): |out - ref| <= 2e-2 + 1e-2 |ref| elementwise,
|lse - ref| <= 1e-3 (base-2 LSE), rows that see no key exactly 0 / -inf.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs

pytestmark = pytest.mark.gpu

ABS, REL, LSE_TOL = 2e-2, 1e-2, 1e-3
FIELDS = ("q_nope", "q_pe", "ckv_cache", "kpe_cache", "qo_indptr", "kv_indptr", "kv_indices")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(case):
    t = [getattr(case, k).to("cuda") for k in FIELDS]
    out = torch.full_like(t[0], float("nan"))
    lse = torch.full(t[0].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pkv.mla_paged_prefill(*t, case.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def run_oracle(case):
    return oracle.mla_prefill(*(getattr(case, k) for k in FIELDS), case.sm_scale)


def check(o, l, ro, rl, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ro)
    bad = err > ABS + REL * np.abs(ro)
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, max abs {err.max()}"
    both = np.isneginf(l) & np.isneginf(rl)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both are -inf: masked out here
        lerr = np.where(both, 0.0, np.abs(l - rl))
    assert np.all(np.isfinite(lerr)) and lerr.max(initial=0) <= LSE_TOL, f"{what}: lse err {lerr.max()}"
    return float(err.max(initial=0)), float(lerr.max(initial=0))


def test_mla_prefill_b8_full():
    case = inputs.mla_prefill_b8()
    say(f"mla_prefill_b8: total_q={case.total_q} pages={case.num_pages}")
    o, l = run_gpu(case)
    ro, rl = run_oracle(case)
    e, le = check(o, l, ro, rl, "mla_prefill_b8")
    say(f"  max abs err {e:.3e}, lse err {le:.3e}")


@pytest.mark.parametrize("q_lens,prefixes", [
    ([1], [0]),
    ([1, 2, 3, 4, 5], [0, 1, 31, 32, 33]),
    ([4, 33, 64, 65], [100, 0, 7, 31]),
    ([130, 9], [2, 500]),
])
def test_mla_edge_lengths(q_lens, prefixes):
    say(f"mla edge q_lens={q_lens} prefixes={prefixes}")
    case = inputs.make_mla(q_lens, prefixes, seed=sum(q_lens) + len(prefixes), extra_pages=5)
    o, l = run_gpu(case)
    ro, rl = run_oracle(case)
    check(o, l, ro, rl, "edge")


@pytest.mark.parametrize("n_batch,seed", [(48, 21), (512, 22), (513, 24), (2000, 23)])
def test_mla_many_batches(n_batch, seed):
    """Many batches, some without query rows, several with equal KV lengths: the tile order
    (batches by KV length, ties by index, in chunks of 512 batches) must still cover every
    row exactly once."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(0, 20 if n_batch < 100 else 4, n_batch)
    q_lens[::7] = 0
    kv_lens = rng.choice([9, 40, 40, 77, 130], n_batch) + q_lens  # repeated lengths -> ties
    kv_lens[1::5] = kv_lens[0]
    prefixes = np.maximum(kv_lens - q_lens, 0)
    say(f"mla many batches: B={n_batch} total_q={int(q_lens.sum())}")
    case = inputs.make_mla(q_lens.tolist(), prefixes.tolist(), seed=seed, extra_pages=3)
    o, l = run_gpu(case)
    ro, rl = run_oracle(case)
    check(o, l, ro, rl, f"B={n_batch}")


def test_mla_empty_kv_and_canaries():
    """A batch with rows but no keys gives 0 / -inf; pages nobody references hold NaN."""
    base = inputs.make_mla([5, 3], [20, 0], seed=9, extra_pages=7)
    # insert a middle batch with 3 rows and no keys
    qo = base.qo_indptr.tolist()
    kv = base.kv_indptr.tolist()
    qo_new = torch.tensor([0, qo[1], qo[1] + 3, qo[2] + 3], dtype=torch.int32)
    kv_new = torch.tensor([0, kv[1], kv[1], kv[2]], dtype=torch.int32)
    pad = lambda t: torch.cat([t[:qo[1]], torch.randn((3,) + t.shape[1:]).to(t.dtype), t[qo[1]:]])
    case = inputs.MlaCase(name="empty_kv", q_nope=pad(base.q_nope), q_pe=pad(base.q_pe),
                          ckv_cache=base.ckv_cache.clone(), kpe_cache=base.kpe_cache.clone(),
                          qo_indptr=qo_new, kv_indptr=kv_new, kv_indices=base.kv_indices, sm_scale=base.sm_scale)
    used = set(case.kv_indices.tolist())
    unused = [i for i in range(case.num_pages) if i not in used]
    assert unused
    case.ckv_cache[unused] = float("nan")
    case.kpe_cache[unused] = float("nan")
    o, l = run_gpu(case)
    ro, rl = run_oracle(case)
    check(o, l, ro, rl, "empty kv + canaries")
    rows = slice(qo[1], qo[1] + 3)
    assert np.all(o[rows] == 0.0) and np.all(np.isneginf(l[rows]))


def test_mla_deterministic():
    case = inputs.make_mla([40, 7], [300, 12], seed=3)
    o1, l1 = run_gpu(case)
    o2, l2 = run_gpu(case)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --------------------------------------------------------------------------------------
# Pages of several tokens (mla_paged_prefill_pages)
# --------------------------------------------------------------------------------------

def run_gpu_paged(case, nan_tail=False):
    t = [getattr(case, k).to("cuda") for k in FIELDS]
    if nan_tail:  # slots past each batch's last token, and unowned pages, hold NaN
        ckv, kpe = t[2].clone(), t[3].clone()
        owned = torch.zeros(case.num_pages, case.page_size, dtype=torch.bool)
        kv = case.kv_indptr.tolist()
        idx = case.kv_indices.tolist()
        last = case.kv_last_page_len.tolist()
        for b in range(case.batch):
            for j in range(kv[b], kv[b + 1]):
                owned[idx[j], : (last[b] if j == kv[b + 1] - 1 else case.page_size)] = True
        mask = (~owned).to("cuda")
        ckv[mask] = float("nan")
        kpe[mask] = float("nan")
        t[2], t[3] = ckv, kpe
    out = torch.full_like(t[0], float("nan"))
    lse = torch.full(t[0].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pkv.mla_paged_prefill(*t, case.sm_scale, out=out, lse=lse, kv_last_page_len=case.kv_last_page_len.to("cuda"))
    torch.cuda.synchronize()
    return out.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def run_oracle_paged(case):
    return oracle.mla_prefill(*(getattr(case, k) for k in FIELDS), case.sm_scale,
                              kv_last_page_len=case.kv_last_page_len)


@pytest.mark.parametrize("page_size", [1, 2, 16, 64])
def test_mla_multi_token_pages(page_size):
    case = inputs.make_mla_paged([5, 40, 1, 17, 3, 0], [30, 0, 100, 7, 64, 9], page_size, seed=page_size)
    say(f"mla pages: page_size={page_size} total_q={case.total_q} pages={case.num_pages}")
    o, l = run_gpu_paged(case)
    ro, rl = run_oracle_paged(case)
    check(o, l, ro, rl, f"page_size={page_size}")
    o2, l2 = run_gpu_paged(case, nan_tail=True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), "slots past the last token leaked into the output"


@pytest.mark.timeout(300)
def test_mla_pages_many_batches():
    """3,000 batches over 16-token pages (some without keys or rows): the token-offset scan
    runs over several passes and every batch's rows still land in place."""
    rng = np.random.default_rng(77)
    B = 3000
    q_lens = rng.integers(0, 4, B)
    prefixes = rng.integers(0, 60, B)
    prefixes[::11] = 0
    q_lens[::11] = 0   # no keys and no rows
    case = inputs.make_mla_paged(q_lens.tolist(), prefixes.tolist(), 16, seed=78)
    say(f"mla pages, many batches: B={B} total_q={case.total_q} pages={case.num_pages}")
    o, l = run_gpu_paged(case)
    ro, rl = run_oracle_paged(case)
    check(o, l, ro, rl, f"B={B} page_size=16")


def test_mla_prefill_b8_pages_of_16():
    """The benchmarked MLA batch's shapes (q_len U[1,512], prefix U[0,4096]) over 16-token pages."""
    case = inputs.mla_prefill_b8_pages(16)
    say(f"mla_prefill_b8 over 16-token pages: total_q={case.total_q} pages={case.num_pages}")
    o, l = run_gpu_paged(case)
    ro, rl = run_oracle_paged(case)
    e, le = check(o, l, ro, rl, "b8 pages of 16")
    say(f"  max abs err {e:.3e}, lse err {le:.3e}")


def test_mla_decode_shapes():
    """One new token per sequence (q_len 1): every key is visible."""
    case = inputs.mla_decode_b64()
    say(f"mla decode shapes: batch={case.batch} pages={case.num_pages}")
    o, l = run_gpu(case)
    ro, rl = run_oracle(case)
    e, le = check(o, l, ro, rl, "mla decode b64")
    say(f"  max abs err {e:.3e}, lse err {le:.3e}")


# --------------------------------------------------------------------------------------
# MLA decode, split-K (mla_paged_decode): the oracle is the prefill oracle with q_len 1
# --------------------------------------------------------------------------------------

def run_decode_gpu(case, split, max_kv_len=None):
    """Both forms of the call: two launches, then one launch (counters) twice on the same
    counters, which must come back zero and give the two-launch result bit for bit (the
    combine is the same code, only its loads differ)."""
    t = {k: getattr(case, k).to("cuda") for k in FIELDS}
    out, lse = pkv.mla_paged_decode(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], t["kv_indptr"],
                                    t["kv_indices"], case.sm_scale, split_tokens=split, max_kv_len=max_kv_len)
    torch.cuda.synchronize()
    B = case.kv_indptr.numel() - 1
    counters = torch.zeros(B, dtype=torch.int32, device="cuda")
    for rep in range(2):
        o1 = torch.full_like(out, float("nan"))
        l1 = torch.full_like(lse, float("nan"))
        pkv.mla_paged_decode(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], t["kv_indptr"], t["kv_indices"],
                             case.sm_scale, split_tokens=split, max_kv_len=max_kv_len, out=o1, lse=l1,
                             counters=counters)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0, "counters not reset"
        assert torch.equal(o1, out) and torch.equal(l1, lse), f"one launch differs from two (call {rep})"
    return out.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


@pytest.mark.parametrize("split", [16, 48, 256, 4096])
def test_mla_split_decode_edges(split):
    """Edge lengths (0, 1, 15, 16, 17, ...) against the oracle, for splits from one key
    group to the whole sequence."""
    kv = [0, 1, 15, 16, 17, 100, 255, 256, 257, 1000, 2049]
    case = inputs.make_mla(np.ones(len(kv), dtype=np.int64), np.maximum(np.array(kv) - 1, 0), seed=split,
                           extra_pages=5)
    # kv_len 0: the generator gives every batch one query token, so build that batch's keys empty
    kvp = case.kv_indptr.clone()
    kvp[1:] = torch.cumsum(torch.tensor([max(k, 0) for k in kv], dtype=torch.int32), 0)
    idx = case.kv_indices[: int(kvp[-1])]
    case = inputs.MlaCase(name="mla_decode_edges", q_nope=case.q_nope, q_pe=case.q_pe, ckv_cache=case.ckv_cache,
                          kpe_cache=case.kpe_cache, qo_indptr=case.qo_indptr, kv_indptr=kvp, kv_indices=idx,
                          sm_scale=case.sm_scale)
    say(f"mla split decode: split={split} kv_lens={kv}")
    o, l = run_decode_gpu(case, split)
    ro, rl = run_oracle(case)
    check(o, l, ro, rl, f"split={split}")
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0])), "empty batch"


@pytest.mark.parametrize("n_batch,split", [(300, 64), (256, 48), (257, 48)])
def test_mla_split_decode_batch_mapping(n_batch, split):
    """Up to 256 batches the kernel packs the non-empty (split, batch) items onto the lowest
    workgroup ids after an in-workgroup scan of the lengths; past 256 it maps workgroups
    split-major. Both against the oracle, with empty batches and ragged lengths."""
    rng = np.random.default_rng(n_batch + split)
    kv = rng.integers(0, 300, n_batch)
    kv[::9] = 0
    kv[1::17] = split  # exactly one split
    case = inputs.make_mla(np.ones(n_batch, dtype=np.int64), np.maximum(kv - 1, 0), seed=n_batch, extra_pages=3)
    kvp = case.kv_indptr.clone()
    kvp[1:] = torch.cumsum(torch.tensor(kv, dtype=torch.int32), 0)
    idx = case.kv_indices[: int(kvp[-1])]
    case = inputs.MlaCase(name="mla_decode_batches", q_nope=case.q_nope, q_pe=case.q_pe, ckv_cache=case.ckv_cache,
                          kpe_cache=case.kpe_cache, qo_indptr=case.qo_indptr, kv_indptr=kvp, kv_indices=idx,
                          sm_scale=case.sm_scale)
    say(f"mla split decode: batches={n_batch} split={split}")
    o, l = run_decode_gpu(case, split)
    ro, rl = run_oracle(case)
    check(o, l, ro, rl, f"batches={n_batch} split={split}")
    empty = np.flatnonzero(kv == 0)
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(l[empty])), "empty batches"


@pytest.mark.parametrize("split", [256, None])
def test_mla_split_decode_b64(split):
    case = inputs.mla_decode_b64()
    say(f"mla split decode b64: pages={case.num_pages} split={split}")
    o, l = run_decode_gpu(case, split)
    ro, rl = run_oracle(case)
    e, le = check(o, l, ro, rl, "split decode b64")
    o2, l2 = run_gpu(case)  # the prefill kernel with q_len 1: the same values within bf16
    check(o, l, o2, l2, "split decode vs prefill kernel")
    say(f"  max abs err {e:.3e}, lse err {le:.3e}")


def test_mla_decode_lengths_past_max_kv_len_stay_in_bounds():
    """A kv_len above the max_kv_len the call promises (a broken contract) is cut to the
    launched splits (len_cap = launched splits x split_tokens): partial rows past them stay
    untouched (NaN here, in arrays wider than the launch), the long sequence's output is
    attention over its first len_cap keys, and the other sequences are unaffected; both
    forms of the call."""
    kv = [100, 700, 40]
    split, max_kv = 128, 300  # 3 splits launched, len_cap 384
    case = inputs.make_mla(np.ones(3, dtype=np.int64), np.array(kv) - 1, seed=41, extra_pages=4)
    t = {k: getattr(case, k).to("cuda") for k in FIELDS}
    cap = 384
    P = 6
    for fused in (False, True):
        acc = torch.full((3, 16, P, 512), float("nan"), dtype=torch.float32, device="cuda")
        m = torch.full((3, 16, P), float("nan"), dtype=torch.float32, device="cuda")
        l = torch.full((3, 16, P), float("nan"), dtype=torch.float32, device="cuda")
        ctr = torch.zeros(3, dtype=torch.int32, device="cuda") if fused else None
        say(f"mla decode past max_kv_len: fused={fused}")
        out, lse = pkv.mla_paged_decode(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], t["kv_indptr"],
                                        t["kv_indices"], case.sm_scale, split_tokens=split, max_kv_len=max_kv,
                                        partials=(acc, m, l), counters=ctr)
        torch.cuda.synchronize()
        assert torch.isnan(m[:, :, 3:]).all() and torch.isnan(acc[:, :, 3:]).all(), "rows past the launched splits"
        o = out.cpu().to(torch.float64).numpy()
        ls = lse.cpu().to(torch.float64).numpy()
        ro, rl = run_oracle(case)
        check(o[[0, 2]], ls[[0, 2]], ro[[0, 2]], rl[[0, 2]], "untouched sequences")
        # the long sequence: its first `cap` keys
        kvp = case.kv_indptr.tolist()
        idx = torch.cat([case.kv_indices[kvp[1]:kvp[1] + cap]])
        cut = inputs.MlaCase(name="cut", q_nope=case.q_nope[1:2], q_pe=case.q_pe[1:2], ckv_cache=case.ckv_cache,
                             kpe_cache=case.kpe_cache, qo_indptr=torch.tensor([0, 1], dtype=torch.int32),
                             kv_indptr=torch.tensor([0, cap], dtype=torch.int32), kv_indices=idx,
                             sm_scale=case.sm_scale)
        co, cl = run_oracle(cut)
        check(o[1:2], ls[1:2], co, cl, "long sequence cut to len_cap")


def test_mla_pool_past_2_25_pages():
    """Pools of more than 2^25 pages: a kpe row's byte offset (page x 128) no longer fits in
    32 bits, so both MLA kernels move the kpe rows one transfer per key instead of one per
    eight keys. A small batch is placed at page ids above 2^25 of a 34 GB pool (only the rows
    it uses are written); the prefill and the split-K decode must match the oracle, and the
    same batch on a small pool bit for bit."""
    case = inputs.make_mla(np.array([1, 37, 5, 64]), np.array([300, 0, 900, 33]), seed=47, extra_pages=7)
    big = (1 << 25) + 4096
    shift = (1 << 25) + 1000
    assert int(case.kv_indices.max()) + shift < big
    small = {k: getattr(case, k).to("cuda") for k in FIELDS}
    say(f"mla pool past 2^25 pages: {big} pages, batch of {case.kv_indptr.numel() - 1}")
    ckv = torch.empty((big, 1, 512), dtype=torch.bfloat16, device="cuda")
    kpe = torch.empty((big, 1, 64), dtype=torch.bfloat16, device="cuda")
    try:
        rows = torch.arange(case.ckv_cache.shape[0], device="cuda") + shift
        ckv.index_copy_(0, rows, small["ckv_cache"])
        kpe.index_copy_(0, rows, small["kpe_cache"])
        idx = small["kv_indices"] + shift
        # prefill
        out_s = torch.full_like(small["q_nope"], float("nan"))
        lse_s = torch.full(small["q_nope"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        pkv.mla_paged_prefill(small["q_nope"], small["q_pe"], small["ckv_cache"], small["kpe_cache"],
                              small["qo_indptr"], small["kv_indptr"], small["kv_indices"], case.sm_scale,
                              out=out_s, lse=lse_s)
        out_b = torch.full_like(out_s, float("nan"))
        lse_b = torch.full_like(lse_s, float("nan"))
        pkv.mla_paged_prefill(small["q_nope"], small["q_pe"], ckv, kpe, small["qo_indptr"], small["kv_indptr"], idx,
                              case.sm_scale, out=out_b, lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(out_b, out_s) and torch.equal(lse_b, lse_s), "prefill: large pool differs from small"
        ro, rl = run_oracle(case)
        check(out_b.cpu().double().numpy(), lse_b.cpu().double().numpy(), ro, rl, "prefill, pool past 2^25 pages")
        # split-K decode: the last query token of each batch, over all of that batch's keys
        last = (small["qo_indptr"][1:] - 1).long()
        q_nope, q_pe = small["q_nope"][last].contiguous(), small["q_pe"][last].contiguous()
        o1, l1 = pkv.mla_paged_decode(q_nope, q_pe, small["ckv_cache"], small["kpe_cache"], small["kv_indptr"],
                                      small["kv_indices"], case.sm_scale, split_tokens=128)
        o2, l2 = pkv.mla_paged_decode(q_nope, q_pe, ckv, kpe, small["kv_indptr"], idx, case.sm_scale,
                                      split_tokens=128)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "decode: large pool differs from small"
        # the decode's token sees every key of its batch: the prefill rows of the last tokens
        # (each batch's last query row is its last position) are the same computation
        check(o2.cpu().double().numpy(), l2.cpu().double().numpy(), ro[last.cpu().numpy()],
              rl[last.cpu().numpy()], "decode, pool past 2^25 pages")
    finally:
        del ckv, kpe
        torch.cuda.empty_cache()
