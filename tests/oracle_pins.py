"""Pins for the float64 oracle: checks against values the oracle does not compute itself.

Each ``pin_*`` takes an oracle module ``orc`` (the real one, or a mutant with a planted
mistake built by ``test_oracle_mutations.py``) and raises AssertionError when the oracle
disagrees with:
  * hand-worked closed-form fixtures under tests/golden/ (each states its derivation);
  * dense brute force on logical (unpaged) K/V that the pin scatters into a pool with its
    own explicit loops, evaluated with library routines (scipy softmax / logsumexp,
    torch repeat_interleave for the head grouping, torch SDPA for MLA);
  * closed forms for special cases (constant V, one token, zero query);
  * invariants (page permutation, split count, trailing sentinels, causal perturbation).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special as sps
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), f"{what}: non-finite mismatch"
    assert diff.max(initial=0.0) <= tol * (1.0 + np.abs(np.where(both_inf, 0, b)).max(initial=0.0)), \
        f"{what}: max diff {diff.max()}"


# ----------------------------------------------------------------------------------------
# Independent construction of paged pools (explicit per-element loops over the layouts)
# ----------------------------------------------------------------------------------------

def scatter_pool(logical_k, logical_v, lens, block_size, num_blocks, layout, x=4, rng=None,
                 fill=np.nan):
    """Scatter per-sequence K/V [KVH, n, D] into a paged pool, one element at a time.

    Token-major K/V: pool[blk, h, slot, d]. x-packed K: pool[blk, h, d // x, slot, d % x];
    x-packed V: pool[blk, h, d, slot]. Pages are handed out by a random permutation.
    Every slot never written stays ``fill`` (NaN), so a gather that touches one shows up.
    """
    rng = rng if rng is not None else np.random.default_rng(123)
    S = len(lens)
    kvh, _, D = logical_k[0].shape
    pages = [-(-int(n) // block_size) for n in lens]
    perm = rng.permutation(num_blocks)
    width = max(1, max(pages))
    bt = np.full((S, width), -1, dtype=np.int64)
    cur = 0
    for b in range(S):
        bt[b, :pages[b]] = perm[cur:cur + pages[b]]
        cur += pages[b]
    if layout == "token_major":
        kc = np.full((num_blocks, kvh, block_size, D), fill)
        vc = np.full((num_blocks, kvh, block_size, D), fill)
    else:
        kc = np.full((num_blocks, kvh, D // x, block_size, x), fill)
        vc = np.full((num_blocks, kvh, D, block_size), fill)
    for b in range(S):
        for t in range(int(lens[b])):
            blk = bt[b, t // block_size]
            slot = t % block_size
            for h in range(kvh):
                for d in range(D):
                    if layout == "token_major":
                        kc[blk, h, slot, d] = logical_k[b][h, t, d]
                        vc[blk, h, slot, d] = logical_v[b][h, t, d]
                    else:
                        kc[blk, h, d // x, slot, d % x] = logical_k[b][h, t, d]
                        vc[blk, h, d, slot] = logical_v[b][h, t, d]
    return kc, vc, bt


def _random_logical(rng, lens, kvh, D):
    K = [rng.standard_normal((kvh, int(n), D)) for n in lens]
    V = [rng.standard_normal((kvh, int(n), D)) for n in lens]
    return K, V


def _brute_decode(q, K, V, lens, scale, G):
    """Dense reference: expand kv heads to query heads with repeat_interleave, then
    scipy softmax / logsumexp per head."""
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    lse = np.full((S, H), -np.inf)
    for b in range(S):
        if int(lens[b]) == 0:
            continue
        Ke = torch.repeat_interleave(torch.from_numpy(K[b]), G, dim=0).numpy()
        Ve = torch.repeat_interleave(torch.from_numpy(V[b]), G, dim=0).numpy()
        for h in range(H):
            logits = scale * np.einsum("td,d->t", Ke[h], q[b, h])
            out[b, h] = sps.softmax(logits) @ Ve[h]
            lse[b, h] = sps.logsumexp(logits)
    return out, lse


def _tiny_case(seed, lens, H, KVH, D, bs, layout, num_blocks=None, x=4):
    rng = np.random.default_rng(seed)
    K, V = _random_logical(rng, lens, KVH, D)
    pages = sum(-(-int(n) // bs) for n in lens)
    nb = num_blocks if num_blocks is not None else pages + 3
    kc, vc, bt = scatter_pool(K, V, lens, bs, nb, layout, x=x, rng=rng)
    q = rng.standard_normal((len(lens), H, D))
    return q, kc, vc, bt, np.asarray(lens), K, V


# ----------------------------------------------------------------------------------------
# Decode pins
# ----------------------------------------------------------------------------------------

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _xpack_from_token_major(kc_tm, vc_tm, x):
    nb, kvh, bs, D = kc_tm.shape
    kc = np.empty((nb, kvh, D // x, bs, x))
    vc = np.empty((nb, kvh, D, bs))
    for blk in range(nb):
        for h in range(kvh):
            for s in range(bs):
                for d in range(D):
                    kc[blk, h, d // x, s, d % x] = kc_tm[blk, h, s, d]
                    vc[blk, h, d, s] = vc_tm[blk, h, s, d]
    return kc, vc


def pin_decode_worked_example(orc):
    g = _load("decode_worked_example.json")
    q = np.array(g["query"])
    kc = np.array(g["key_cache_token_major"])
    vc = np.array(g["value_cache_token_major"])
    bt = np.array(g["block_tables"])
    lens = np.array(g["seq_lens"])
    exp_out = np.array(g["expected_out"])
    exp_lse = np.array(g["expected_lse"])
    kx, vx = _xpack_from_token_major(kc, vc, 2)
    for layout, k, v in (("token_major", kc, vc), ("xpacked", kx, vx)):
        out, lse = orc.decode(q, k, v, layout, bt, lens, g["scale"], g["num_kv_heads"], g["block_size"])
        _close(out, exp_out, what=f"worked out {layout}")
        _close(lse, exp_lse, what=f"worked lse {layout}")
        acc, m, l = orc.decode_partials(q, k, v, layout, bt, lens, g["scale"], g["num_kv_heads"],
                                        g["block_size"], g["partition_size"], g["max_num_partitions"])
        em = np.array([[[(-np.inf if z is None else z) for z in row] for row in b] for b in g["expected_partial_m"]])
        _close(m, em, what="worked partial m")
        _close(l, np.array(g["expected_partial_l"]), what="worked partial l")
        for h in range(2):
            for p in range(2):
                _close(acc[0, h, p], np.array(g["expected_partial_acc"][0][h][p]), what="worked partial acc")
        out2, lse2 = orc.reduce_partials(acc, m, l, lens, g["partition_size"])
        _close(out2, exp_out, what="worked reduce out")
        _close(lse2, exp_lse, what="worked reduce lse")


def pin_reduce_worked_example(orc):
    """Reduce on hand-set partials: m=[0, ln3], l=[1, 1] -> weights 1/4, 3/4."""
    acc = np.zeros((1, 1, 3, 2))
    acc[0, 0, 0] = [4.0, 0.0]
    acc[0, 0, 1] = [0.0, 8.0]
    acc[0, 0, 2] = [np.nan, np.nan]        # sentinel partition: must never be read
    m = np.array([[[0.0, math.log(3.0), -np.inf]]])
    l = np.array([[[1.0, 1.0, 0.0]]])
    out, lse = orc.reduce_partials(acc, m, l, np.array([7]), 4)   # ceil(7/4) = 2 partitions
    _close(out[0, 0], [1.0, 6.0], what="reduce worked out")
    _close(lse[0, 0], math.log(4.0), what="reduce worked lse")


def pin_decode_brute_force(orc):
    """Dense brute force on logical K/V, both layouts, several G, block sizes, tails."""
    shapes = [  # lens, H, KVH, D, bs
        ([5, 0, 33], 4, 2, 8, 4),
        ([1, 17, 16], 3, 1, 8, 16),     # MQA, G=3
        ([9, 2], 2, 2, 4, 2),           # MHA
        ([40], 6, 2, 8, 16),            # G=3, several pages with a tail
        ([3, 12, 31], 8, 2, 8, 1),      # block_size 1
    ]
    for i, (lens, H, KVH, D, bs) in enumerate(shapes):
        for layout in ("token_major", "xpacked"):
            q, kc, vc, bt, lens_a, K, V = _tiny_case(100 + i, lens, H, KVH, D, bs, layout)
            scale = 0.37 + 0.1 * i
            out, lse = orc.decode(q, kc, vc, layout, bt, lens_a, scale, KVH, bs)
            ref_out, ref_lse = _brute_decode(q, K, V, lens_a, scale, H // KVH)
            _close(out, ref_out, 1e-12, what=f"brute out {i} {layout}")
            _close(lse, ref_lse, 1e-12, what=f"brute lse {i} {layout}")


def pin_decode_special_cases(orc):
    rng = np.random.default_rng(7)
    lens = [1, 23, 48]
    H, KVH, D, bs = 4, 2, 8, 16
    q, kc, vc, bt, lens_a, K, V = _tiny_case(7, lens, H, KVH, D, bs, "token_major")
    # constant V = c  ->  out = c for every head
    c = rng.standard_normal(D)
    Vc = [np.broadcast_to(c, v.shape).copy() for v in V]
    kc2, vc2, bt2 = scatter_pool(K, Vc, lens, bs, kc.shape[0], "token_major", rng=np.random.default_rng(9))
    out, _ = orc.decode(q, kc2, vc2, "token_major", bt2, lens_a, 0.5, KVH, bs)
    for b in range(3):
        for h in range(H):
            _close(out[b, h], c, 1e-12, what="constant V")
    # len = 1  ->  out = v_0 and lse = scale * q . k_0
    out, lse = orc.decode(q, kc, vc, "token_major", bt, lens_a, 0.5, KVH, bs)
    for h in range(H):
        _close(out[0, h], V[0][h // 2, 0], 1e-12, what="len 1 out")
        _close(lse[0, h], 0.5 * float(np.dot(q[0, h], K[0][h // 2, 0])), 1e-12, what="len 1 lse")
    # q = 0  ->  out = mean of the value rows, lse = ln n
    out, lse = orc.decode(np.zeros_like(q), kc, vc, "token_major", bt, lens_a, 0.5, KVH, bs)
    for b in range(3):
        for h in range(H):
            _close(out[b, h], V[b][h // 2].mean(axis=0), 1e-12, what="q=0 mean")
            _close(lse[b, h], math.log(lens[b]), 1e-12, what="q=0 lse")


def pin_split_invariance(orc):
    lens = [1, 16, 37, 100, 0]
    H, KVH, D, bs = 6, 3, 8, 4
    for layout in ("token_major", "xpacked"):
        q, kc, vc, bt, lens_a, K, V = _tiny_case(11, lens, H, KVH, D, bs, layout)
        out, lse = orc.decode(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs)
        for ps in (1, 2, 3, 4, 8, 12, 64, 100, 130):
            P = -(-max(lens) // ps) + 2
            acc, m, l = orc.decode_partials(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs, ps, P)
            o2, lse2 = orc.reduce_partials(acc, m, l, lens_a, ps)
            _close(o2, out, 1e-12, what=f"split ps={ps}")
            _close(lse2, lse, 1e-12, what=f"split lse ps={ps}")


def pin_partition_stats(orc):
    """Each partition's (m, l, acc) against scipy on that partition's own scores."""
    lens = [45, 9]
    H, KVH, D, bs, ps = 4, 2, 8, 4, 16
    q, kc, vc, bt, lens_a, K, V = _tiny_case(13, lens, H, KVH, D, bs, "xpacked")
    scale = 0.8
    acc, m, l = orc.decode_partials(q, kc, vc, "xpacked", bt, lens_a, scale, KVH, bs, ps, 4)
    for b, n in enumerate(lens):
        Ke = torch.repeat_interleave(torch.from_numpy(K[b]), 2, dim=0).numpy()
        Ve = torch.repeat_interleave(torch.from_numpy(V[b]), 2, dim=0).numpy()
        for h in range(H):
            s_all = scale * np.einsum("td,d->t", Ke[h], q[b, h])
            for p in range(4):
                t0, t1 = p * ps, min((p + 1) * ps, n)
                if t0 >= n:
                    assert m[b, h, p] == -np.inf and l[b, h, p] == 0.0, "sentinel"
                    continue
                sp = s_all[t0:t1]
                _close(m[b, h, p], sp.max(), 1e-12, what="partition max")
                _close(m[b, h, p] + math.log(l[b, h, p]), sps.logsumexp(sp), 1e-12, what="partition lse")
                _close(acc[b, h, p] / l[b, h, p], sps.softmax(sp) @ Ve[h][t0:t1], 1e-12,
                       what="partition normalized acc")


def pin_sentinel_padding(orc):
    """Extra trailing sentinel partitions leave the reduce unchanged, bit for bit."""
    lens = [30, 5]
    q, kc, vc, bt, lens_a, K, V = _tiny_case(17, lens, 2, 1, 8, 4, "token_major")
    a1, m1, l1 = orc.decode_partials(q, kc, vc, "token_major", bt, lens_a, 1.0, 1, 4, 8, 4)
    a2, m2, l2 = orc.decode_partials(q, kc, vc, "token_major", bt, lens_a, 1.0, 1, 4, 8, 9)
    assert np.all(m2[:, :, 4:] == -np.inf) and np.all(l2[:, :, 4:] == 0.0)
    assert np.all(m2[1, :, 1:] == -np.inf) and np.all(l2[1, :, 1:] == 0.0)
    a2[:, :, 4:] = np.nan      # a reduce that reads past P_b turns this into NaN
    a2[1, :, 1:] = np.nan
    o1, s1 = orc.reduce_partials(a1, m1, l1, lens_a, 8)
    o2, s2 = orc.reduce_partials(a2, m2, l2, lens_a, 8)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def pin_page_permutation(orc):
    """Permuting the pool's block axis (tables remapped) changes nothing, bit for bit."""
    lens = [21, 50, 7]
    for layout in ("token_major", "xpacked"):
        q, kc, vc, bt, lens_a, K, V = _tiny_case(19, lens, 4, 2, 8, 4, layout)
        out, lse = orc.decode(q, kc, vc, layout, bt, lens_a, 0.7, 2, 4)
        perm = np.random.default_rng(5).permutation(kc.shape[0])
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm))
        bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1)
        out2, lse2 = orc.decode(q, kc[perm], vc[perm], layout, bt2, lens_a, 0.7, 2, 4)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2), "page permutation"


def pin_empty_sequence(orc):
    lens = [0, 3]
    q, kc, vc, bt, lens_a, K, V = _tiny_case(23, lens, 2, 1, 4, 2, "token_major")
    out, lse = orc.decode(q, kc, vc, "token_major", bt, lens_a, 1.0, 1, 2)
    assert np.all(out[0] == 0.0) and np.all(lse[0] == -np.inf)
    acc, m, l = orc.decode_partials(q, kc, vc, "token_major", bt, lens_a, 1.0, 1, 2, 2, 2)
    assert np.all(m[0] == -np.inf) and np.all(l[0] == 0.0)
    o2, s2 = orc.reduce_partials(acc, m, l, lens_a, 2)
    assert np.all(o2[0] == 0.0) and np.all(s2[0] == -np.inf)


# NUM_SPLITS policy of the flash-decode post's partial kernel, worked by hand for a
# 37-token sequence in 4-token pages (nb = ceil(37 / 4) = 10 pages):
#   NS = 1  -> bps = 10 pages -> one range of all 37 tokens
#   NS = 3  -> bps = ceil(10 / 3) = 4 pages = 16 tokens -> [0,16) [16,32) [32,37)
#   NS = 4  -> bps = 3 pages = 12 tokens -> [0,12) [12,24) [24,36) [36,37)
#   NS = 6  -> bps = 2 pages = 8 tokens -> five ranges, split 5 starts at page 10: empty
#   NS = 16 -> bps = 1 page -> ten 4-token ranges (the last [36,37)), splits 10..15 empty
# and for a 5-token sequence (nb = 2): NS = 4 -> bps = 1 -> [0,4) [4,5), splits 2, 3 empty.
SPLIT_POLICY_CASES = {
    (37, 1): [(0, 37)],
    (37, 3): [(0, 16), (16, 32), (32, 37)],
    (37, 4): [(0, 12), (12, 24), (24, 36), (36, 37)],
    (37, 6): [(0, 8), (8, 16), (16, 24), (24, 32), (32, 37)],
    (37, 16): [(4 * i, min(4 * i + 4, 37)) for i in range(10)],
    (5, 4): [(0, 4), (4, 5)],
}


def _check_partition_stats(acc, m, l, b, h, s_all, Ve_h, ranges, P, normalized, what):
    for p in range(P):
        if p >= len(ranges):
            assert m[b, h, p] == -np.inf and l[b, h, p] == 0.0, f"{what}: sentinel at p={p}"
            continue
        t0, t1 = ranges[p]
        sp = s_all[t0:t1]
        _close(m[b, h, p], sp.max(), 1e-12, what=f"{what}: partition max")
        _close(m[b, h, p] + math.log(l[b, h, p]), sps.logsumexp(sp), 1e-12, what=f"{what}: partition lse")
        avg = acc[b, h, p] if normalized else acc[b, h, p] / l[b, h, p]
        _close(avg, sps.softmax(sp) @ Ve_h[t0:t1], 1e-12, what=f"{what}: partition average")


def pin_split_policy(orc):
    """NUM_SPLITS page-aligned splits: the hand-worked ranges above, their sentinels, and the
    reduce against dense brute force for every split count."""
    H, KVH, D, bs, scale = 4, 2, 8, 4, 0.6
    for (n, ns), ranges in SPLIT_POLICY_CASES.items():
        assert [tuple(r) for r in orc.partition_ranges(n, bs, 0, ns)] == ranges, f"ranges n={n} NS={ns}"
    for layout in ("token_major", "xpacked"):
        q, kc, vc, bt, lens_a, K, V = _tiny_case(29, [37, 5, 0], H, KVH, D, bs, layout)
        ref_out, ref_lse = _brute_decode(q, K, V, lens_a, scale, H // KVH)
        for ns in (1, 2, 3, 4, 6, 7, 10, 16):
            acc, m, l = orc.decode_partials(q, kc, vc, layout, bt, lens_a, scale, KVH, bs, 0, ns,
                                            num_splits=ns)
            for b, n in enumerate((37, 5)):
                ranges = SPLIT_POLICY_CASES.get((n, ns))
                if ranges is None:
                    continue
                Ke = torch.repeat_interleave(torch.from_numpy(K[b]), H // KVH, dim=0).numpy()
                Ve = torch.repeat_interleave(torch.from_numpy(V[b]), H // KVH, dim=0).numpy()
                for h in range(H):
                    s_all = scale * np.einsum("td,d->t", Ke[h], q[b, h])
                    _check_partition_stats(acc, m, l, b, h, s_all, Ve[h], ranges, ns, False,
                                           f"{layout} NS={ns} b={b}")
            assert np.all(m[2] == -np.inf) and np.all(l[2] == 0.0), "empty sequence: all sentinels"
            o2, s2 = orc.reduce_partials(acc, m, l, lens_a, 0, num_splits=ns, block_size=bs)
            _close(o2, ref_out, 1e-12, what=f"{layout} NS={ns} reduce")
            _close(s2, ref_lse, 1e-12, what=f"{layout} NS={ns} reduce lse")


def pin_normalized_partials(orc):
    """PagedAttention V2 form: tmp_output = softmax over the partition's own scores times its
    V rows; exp_sums and max_logits as before; its reduce against dense brute force, with
    NaN in every never-read row."""
    lens = [45, 9, 0, 16]
    H, KVH, D, bs, ps, scale = 6, 2, 8, 4, 16, 0.8
    for layout in ("xpacked", "token_major"):
        q, kc, vc, bt, lens_a, K, V = _tiny_case(31, lens, H, KVH, D, bs, layout)
        acc, m, l = orc.decode_partials(q, kc, vc, layout, bt, lens_a, scale, KVH, bs, ps, 5, normalized=True)
        G = H // KVH
        for b, n in enumerate(lens):
            if n == 0:
                assert np.all(m[b] == -np.inf) and np.all(l[b] == 0.0)
                continue
            Ke = torch.repeat_interleave(torch.from_numpy(K[b]), G, dim=0).numpy()
            Ve = torch.repeat_interleave(torch.from_numpy(V[b]), G, dim=0).numpy()
            ranges = [(t0, min(t0 + ps, n)) for t0 in range(0, n, ps)]
            for h in range(H):
                s_all = scale * np.einsum("td,d->t", Ke[h], q[b, h])
                _check_partition_stats(acc, m, l, b, h, s_all, Ve[h], ranges, 5, True, f"{layout} normalized")
        ref_out, ref_lse = _brute_decode(q, K, V, lens_a, scale, G)
        acc = acc.copy()
        for b, n in enumerate(lens):
            acc[b, :, -(-n // ps):] = np.nan
        o2, s2 = orc.reduce_partials(acc, m, l, lens_a, ps, normalized=True)
        _close(o2, ref_out, 1e-12, what=f"{layout} normalized reduce")
        _close(s2, ref_lse, 1e-12, what=f"{layout} normalized reduce lse")
        # NUM_SPLITS and normalized together
        acc, m, l = orc.decode_partials(q, kc, vc, layout, bt, lens_a, scale, KVH, bs, 0, 3,
                                        num_splits=3, normalized=True)
        o3, s3 = orc.reduce_partials(acc, m, l, lens_a, 0, num_splits=3, block_size=bs, normalized=True)
        _close(o3, ref_out, 1e-12, what=f"{layout} normalized NS=3 reduce")
        _close(s3, ref_lse, 1e-12, what=f"{layout} normalized NS=3 reduce lse")


def pin_alibi_closed_forms(orc):
    """ALiBi against closed forms. With a zero query only the bias remains, so the weights are
    geometric: w_t = r^(n-1-t) / Z with r = e^-m and Z = (1 - r^n) / (1 - r), and
    lse = ln Z. With one token the bias is zero. With two tokens the older one loses m:
    weights e^(s0 - m) and e^s1, worked out here with math.exp."""
    for layout in ("token_major", "xpacked"):
        lens = [1, 2, 7, 30, 0]
        H, KVH, D, bs = 4, 2, 8, 4
        q, kc, vc, bt, lens_a, K, V = _tiny_case(41, lens, H, KVH, D, bs, layout)
        slopes = np.array([0.5, 0.25, 0.125, 0.0625])
        out0, lse0 = orc.decode(np.zeros_like(q), kc, vc, layout, bt, lens_a, 0.7, KVH, bs, alibi_slopes=slopes)
        for b, n in enumerate(lens):
            if n == 0:
                assert np.all(out0[b] == 0.0) and np.all(lse0[b] == -np.inf)
                continue
            for h in range(H):
                r = math.exp(-slopes[h])
                Z = (1.0 - r ** n) / (1.0 - r)
                w = np.array([r ** (n - 1 - t) for t in range(n)]) / Z
                _close(out0[b, h], w @ V[b][h // 2], 1e-12, what=f"alibi zero-query out n={n}")
                _close(lse0[b, h], math.log(Z), 1e-12, what=f"alibi zero-query lse n={n}")
        out, lse = orc.decode(q, kc, vc, layout, bt, lens_a, 0.7, KVH, bs, alibi_slopes=slopes)
        for h in range(H):
            kv = h // 2
            s0 = 0.7 * float(K[0][kv][0] @ q[0, h])      # one token: no bias
            _close(lse[0, h], s0, 1e-12, what="alibi one token lse")
            _close(out[0, h], V[0][kv][0], 1e-12, what="alibi one token out")
            a0 = 0.7 * float(K[1][kv][0] @ q[1, h]) - slopes[h]   # two tokens: the older loses m
            a1 = 0.7 * float(K[1][kv][1] @ q[1, h])
            e0, e1 = math.exp(a0), math.exp(a1)
            _close(out[1, h], (e0 * V[1][kv][0] + e1 * V[1][kv][1]) / (e0 + e1), 1e-12, what="alibi two tokens")
            _close(lse[1, h], math.log(e0 + e1), 1e-12, what="alibi two tokens lse")


def pin_alibi_split_invariance(orc):
    """Partials carry each token's absolute position: any split reduces to the unsplit
    ALiBi result; zero slopes give the plain result bit for bit."""
    lens = [1, 16, 37, 100, 0]
    H, KVH, D, bs = 6, 3, 8, 4
    slopes = np.array([0.3, 0.1, 0.05, 0.02, 0.01, 0.7])
    for layout in ("token_major", "xpacked"):
        q, kc, vc, bt, lens_a, K, V = _tiny_case(43, lens, H, KVH, D, bs, layout)
        out, lse = orc.decode(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs, alibi_slopes=slopes)
        for ps in (4, 12, 64):
            P = -(-max(lens) // ps)
            acc, m, l = orc.decode_partials(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs, ps, P,
                                            alibi_slopes=slopes)
            o2, s2 = orc.reduce_partials(acc, m, l, lens_a, ps)
            _close(o2, out, 1e-12, what=f"alibi split ps={ps}")
            _close(s2, lse, 1e-12, what=f"alibi split lse ps={ps}")
        o0, s0 = orc.decode(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs, alibi_slopes=np.zeros(H))
        o1, s1 = orc.decode(q, kc, vc, layout, bt, lens_a, 0.3, KVH, bs)
        assert np.array_equal(o0, o1) and np.array_equal(s0, s1), "zero slopes"
        # a bias only differences of which matter: out is unchanged by the reference
        # position, so compare against brute force with keys re-weighted by e^-m(n-1-t)
        for b, n in enumerate(lens):
            for h in range(H):
                if n == 0:
                    continue
                logits = 0.3 * (K[b][h // 2] @ q[b, h])
                w = sps.softmax(logits) * np.exp(-slopes[h] * ((n - 1) - np.arange(n)))
                _close(out[b, h], (w / w.sum()) @ V[b][h // 2], 1e-12, what="alibi reweighting")


def pin_quantized_cache(orc):
    """float8 (e4m3) pools: with unit scales the result is dense brute force on the stored
    values; k_scale acts exactly like a factor on the softmax scale (out and lse); v_scale
    multiplies out and leaves lse alone; the same for split partials."""
    lens = [1, 16, 37, 0, 70]
    H, KVH, D, bs = 4, 2, 16, 4  # x-packed fp8 keys: x = 16 one-byte elements per chunk
    for layout in ("token_major", "xpacked"):
        rng = np.random.default_rng(47)
        K = [torch.from_numpy(rng.standard_normal((KVH, n, D))).to(torch.float8_e4m3fn).to(torch.float64).numpy()
             for n in lens]
        V = [torch.from_numpy(rng.standard_normal((KVH, n, D))).to(torch.float8_e4m3fn).to(torch.float64).numpy()
             for n in lens]
        pages = sum(-(-n // bs) for n in lens)
        kc, vc, bt = scatter_pool(K, V, lens, bs, pages + 3, layout, x=16, rng=rng)
        kc8 = torch.from_numpy(kc).to(torch.float8_e4m3fn)
        vc8 = torch.from_numpy(vc).to(torch.float8_e4m3fn)
        q = rng.standard_normal((len(lens), H, D))
        lens_a = np.asarray(lens)
        out, lse = orc.decode(q, kc8, vc8, layout, bt, lens_a, 0.4, KVH, bs)
        ref_out, ref_lse = _brute_decode(q, K, V, lens_a, 0.4, H // KVH)
        _close(out, ref_out, 1e-12, what="fp8 pools, unit scales")
        _close(lse, ref_lse, 1e-12, what="fp8 pools, unit scales lse")
        o_k, s_k = orc.decode(q, kc8, vc8, layout, bt, lens_a, 0.4, KVH, bs, k_scale=0.25)
        o_s, s_s = orc.decode(q, kc8, vc8, layout, bt, lens_a, 0.1, KVH, bs)
        _close(o_k, o_s, 1e-12, what="k_scale as a softmax-scale factor")
        _close(s_k, s_s, 1e-12, what="k_scale as a softmax-scale factor (lse)")
        o_v, s_v = orc.decode(q, kc8, vc8, layout, bt, lens_a, 0.4, KVH, bs, v_scale=3.0)
        _close(o_v, 3.0 * out, 1e-12, what="v_scale multiplies out")
        _close(s_v, lse, 1e-12, what="v_scale leaves lse")
        acc, m, l = orc.decode_partials(q, kc8, vc8, layout, bt, lens_a, 0.4, KVH, bs, 16, 5, k_scale=0.25,
                                        v_scale=3.0)
        o2, s2 = orc.reduce_partials(acc, m, l, lens_a, 16)
        _close(o2, 3.0 * o_s, 1e-12, what="quantized partials")
        _close(s2, s_s, 1e-12, what="quantized partials lse")


# ----------------------------------------------------------------------------------------
# MLA pins
# ----------------------------------------------------------------------------------------

def pin_mla_worked_example(orc):
    g = _load("mla_worked_example.json")
    O, lse2 = orc.mla_prefill(np.array(g["q_nope"]), np.array(g["q_pe"]), np.array(g["ckv_cache"]),
                              np.array(g["kpe_cache"]), np.array(g["qo_indptr"]), np.array(g["kv_indptr"]),
                              np.array(g["kv_indices"]), g["sm_scale"])
    _close(O, np.array(g["expected_out"]), what="mla worked O")
    _close(lse2, np.array(g["expected_lse2"]), what="mla worked lse2")


def _mla_tiny(seed, q_lens, prefixes, H=3, Dc=8, Dp=4, extra=2):
    rng = np.random.default_rng(seed)
    kv_lens = [a + b for a, b in zip(q_lens, prefixes)]
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int64)
    n_pages = int(kv[-1]) + extra
    idx = rng.permutation(n_pages)[: int(kv[-1])]
    T = int(qo[-1])
    qn = rng.standard_normal((T, H, Dc))
    qp = rng.standard_normal((T, H, Dp))
    ckv = rng.standard_normal((n_pages, 1, Dc))
    kpe = rng.standard_normal((n_pages, 1, Dp))
    return qn, qp, ckv, kpe, qo, kv, idx


def _sdpa_rows(qn, qp, ckv, kpe, tok, q_len, sm_scale):
    """torch float64 SDPA on [q_nope|q_pe] x [ckv|kpe] with an explicit bottom-right mask."""
    kv_len = len(tok)
    q = torch.from_numpy(np.concatenate([qn, qp], axis=-1)).permute(1, 0, 2)       # [H, q_len, Dc+Dp]
    kk = torch.from_numpy(np.concatenate([ckv[tok, 0], kpe[tok, 0]], axis=-1))      # [kv_len, Dc+Dp]
    vv = torch.from_numpy(ckv[tok, 0])                                              # [kv_len, Dc]
    H = q.shape[0]
    k = kk.unsqueeze(0).expand(H, -1, -1).contiguous()
    v = vv.unsqueeze(0).expand(H, -1, -1).contiguous()
    i = torch.arange(q_len)[:, None]
    j = torch.arange(kv_len)[None, :]
    mask = j <= (kv_len - q_len) + i
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=sm_scale)
    logits = sm_scale * torch.matmul(q, k.transpose(-1, -2))
    logits = logits.masked_fill(~mask, -math.inf)
    lse2 = torch.logsumexp(logits, dim=-1) / math.log(2.0)
    return o.permute(1, 0, 2).numpy(), lse2.permute(1, 0).numpy()


def pin_mla_sdpa(orc):
    """Ragged batch with permuted page ids against per-batch torch SDPA (float64)."""
    q_lens, prefixes = [3, 1, 7, 4], [5, 0, 0, 11]
    qn, qp, ckv, kpe, qo, kv, idx = _mla_tiny(29, q_lens, prefixes)
    sm = 0.41
    O, lse2 = orc.mla_prefill(qn, qp, ckv, kpe, qo, kv, idx, sm)
    for b in range(len(q_lens)):
        r0, r1 = qo[b], qo[b + 1]
        ro, rl = _sdpa_rows(qn[r0:r1], qp[r0:r1], ckv, kpe, idx[kv[b]:kv[b + 1]], r1 - r0, sm)
        _close(O[r0:r1], ro, 1e-12, what=f"mla sdpa O b={b}")
        _close(lse2[r0:r1], rl, 1e-12, what=f"mla sdpa lse b={b}")


def pin_mla_causal_perturbation(orc):
    q_lens, prefixes = [6], [4]
    qn, qp, ckv, kpe, qo, kv, idx = _mla_tiny(31, q_lens, prefixes, extra=0)
    O, L = orc.mla_prefill(qn, qp, ckv, kpe, qo, kv, idx, 0.5)
    for r in range(6):
        abs_pos = 4 + r
        ck2, kp2 = ckv.copy(), kpe.copy()
        for j in range(abs_pos + 1, 10):
            ck2[idx[j]] += 100.0
            kp2[idx[j]] -= 50.0
        O2, L2 = orc.mla_prefill(qn, qp, ck2, kp2, qo, kv, idx, 0.5)
        assert np.array_equal(O2[r], O[r]) and np.array_equal(L2[r], L[r]), f"future key leaked into row {r}"
        ck3 = ckv.copy()
        ck3[idx[abs_pos]] += 1.0
        O3, _ = orc.mla_prefill(qn, qp, ck3, kpe, qo, kv, idx, 0.5)
        assert not np.array_equal(O3[r], O[r]), f"diagonal key ignored in row {r}"


def pin_mla_special_cases(orc):
    q_lens, prefixes = [5, 2], [3, 0]
    qn, qp, ckv, kpe, qo, kv, idx = _mla_tiny(37, q_lens, prefixes)
    O, L = orc.mla_prefill(np.zeros_like(qn), np.zeros_like(qp), ckv, kpe, qo, kv, idx, 0.9)
    for b in range(2):
        for i in range(q_lens[b]):
            r = qo[b] + i
            vis = prefixes[b] + i + 1
            mean = torch.from_numpy(ckv[idx[kv[b]:kv[b] + vis], 0]).mean(dim=0).numpy()
            for h in range(qn.shape[1]):
                _close(O[r, h], mean, 1e-12, what="mla q=0 mean")
                _close(L[r, h], math.log2(vis), 1e-12, what="mla q=0 lse2")
    # a batch with no keys at all gives zeros and -inf (its rows see nothing)
    qo_e = np.array([0, 2, 2 + q_lens[0]])
    kv_e = np.array([0, 0, kv[1]])
    rows = 2 + q_lens[0]
    qn_e = np.concatenate([np.ones((2,) + qn.shape[1:]), qn[:q_lens[0]]])
    qp_e = np.concatenate([np.ones((2,) + qp.shape[1:]), qp[:q_lens[0]]])
    O, L = orc.mla_prefill(qn_e, qp_e, ckv, kpe, qo_e, kv_e, idx[:kv[1]], 0.9)
    assert O.shape[0] == rows
    assert np.all(O[:2] == 0.0) and np.all(L[:2] == -np.inf)


def paged_mla_pool(ckv1, kpe1, kv_lens, starts, ps, rng, extra_pages=2):
    """Scatter per-batch token rows of a one-token-per-page pool into pages of ps tokens,
    element by element: batch b's token j (row starts[b] + j of ckv1 / kpe1) goes to slot
    j % ps of its (j // ps)-th page; pages are handed out by a random permutation and every
    slot never written stays NaN. Returns (ckv, kpe, kv_indptr in pages, kv_indices,
    kv_last_page_len)."""
    Dc, Dp = ckv1.shape[2], kpe1.shape[2]
    n_pages_b = [-(-int(n) // ps) for n in kv_lens]
    total = sum(n_pages_b) + extra_pages
    perm = rng.permutation(total)
    ckv = np.full((total, ps, Dc), np.nan)
    kpe = np.full((total, ps, Dp), np.nan)
    indptr = [0]
    indices = []
    last = []
    cur = 0
    for b, n in enumerate(kv_lens):
        pages = perm[cur:cur + n_pages_b[b]]
        cur += n_pages_b[b]
        indices.extend(int(x) for x in pages)
        indptr.append(len(indices))
        last.append(int(n) - (n_pages_b[b] - 1) * ps if n_pages_b[b] else ps)
        for j in range(int(n)):
            for d in range(Dc):
                ckv[pages[j // ps], j % ps, d] = ckv1[starts[b] + j, 0, d]
            for d in range(Dp):
                kpe[pages[j // ps], j % ps, d] = kpe1[starts[b] + j, 0, d]
    return ckv, kpe, np.asarray(indptr), np.asarray(indices, dtype=np.int64), np.asarray(last)


def pin_mla_multi_token_pages(orc):
    """Pages of 2, 3, 4 and 16 tokens (last pages partly filled, NaN elsewhere) against
    float64 SDPA over the same tokens laid out one per row."""
    q_lens, prefixes = [3, 1, 7, 4, 2], [5, 0, 0, 11, 30]
    kv_lens = [a + b for a, b in zip(q_lens, prefixes)]
    rng = np.random.default_rng(37)
    H, Dc, Dp = 3, 8, 4
    T = sum(q_lens)
    N = sum(kv_lens)
    qn = rng.standard_normal((T, H, Dc))
    qp = rng.standard_normal((T, H, Dp))
    ckv1 = rng.standard_normal((N, 1, Dc))
    kpe1 = rng.standard_normal((N, 1, Dp))
    qo = np.concatenate([[0], np.cumsum(q_lens)])
    starts = np.concatenate([[0], np.cumsum(kv_lens)])
    sm = 0.37
    for ps in (2, 3, 4, 16):
        ckv, kpe, kvp, idx, last = paged_mla_pool(ckv1, kpe1, kv_lens, starts, ps, rng)
        O, L = orc.mla_prefill(qn, qp, ckv, kpe, qo, kvp, idx, sm, kv_last_page_len=last)
        for b in range(len(q_lens)):
            r0, r1 = qo[b], qo[b + 1]
            tok = np.arange(starts[b], starts[b + 1])
            ro, rl = _sdpa_rows(qn[r0:r1], qp[r0:r1], ckv1, kpe1, tok, r1 - r0, sm)
            _close(O[r0:r1], ro, 1e-12, what=f"mla ps={ps} O b={b}")
            _close(L[r0:r1], rl, 1e-12, what=f"mla ps={ps} lse b={b}")
    # full pages: no last-page array needed
    kv_full = [8, 4]
    st = np.array([0, 8, 12])
    ckv, kpe, kvp, idx, last = paged_mla_pool(ckv1, kpe1, kv_full, st, 4, rng)
    qo2 = np.array([0, 2, 3])
    O, L = orc.mla_prefill(qn[:3], qp[:3], ckv, kpe, qo2, kvp, idx, sm)
    for b in range(2):
        ro, rl = _sdpa_rows(qn[qo2[b]:qo2[b + 1]], qp[qo2[b]:qo2[b + 1]], ckv1, kpe1,
                            np.arange(st[b], st[b + 1]), qo2[b + 1] - qo2[b], sm)
        _close(O[qo2[b]:qo2[b + 1]], ro, 1e-12, what="mla full pages O")
        _close(L[qo2[b]:qo2[b + 1]], rl, 1e-12, what="mla full pages lse")


DECODE_PINS = [pin_decode_worked_example, pin_reduce_worked_example, pin_decode_brute_force,
               pin_decode_special_cases, pin_split_invariance, pin_partition_stats,
               pin_sentinel_padding, pin_page_permutation, pin_empty_sequence, pin_split_policy,
               pin_normalized_partials, pin_alibi_closed_forms, pin_alibi_split_invariance,
               pin_quantized_cache]
MLA_PINS = [pin_mla_worked_example, pin_mla_sdpa, pin_mla_causal_perturbation,
            pin_mla_special_cases, pin_mla_multi_token_pages]
ALL_PINS = DECODE_PINS + MLA_PINS
