"""Oracle for single-token paged-KV GQA decode, unsplit and split-K.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests/, the smoke
entry and bench.py's cpu_baseline leg use it.

Sources (the pages this restates; no code is taken from them):
  * PagedAttention V2 Triton page (``paged_attention_v2_triton.py``):
    ``_partition_attn_kernel`` (paged gather through ``block_tables``, x-packed
    key layout, GQA head grouping, empty-partition sentinel m=-inf / l=0) and
    ``_reduce_partitions_kernel`` (partitions per sequence = ceil(len / ps)).
  * Flash-decode blog post (koas-w, "flashdecode"): token-major K/V layout,
    ``Decode_Paged_GQAAttention_Kernel`` (unsplit online softmax, o / l),
    ``_flash_decode_partial_kernel`` (unnormalized partial accumulator) and
    ``_flash_decode_combine_kernel`` (M = max m_s, f = exp(m_s - M),
    out = sum f * acc_s / sum f * l_s; zeros for an empty context).

Readings taken where the pages differ or are silent:
  partial acc is unnormalized (normalized on request, for the PagedAttention V2
  interface); partial m is in natural-log units of the scaled
  score; partitions are token ranges [p*ps, min((p+1)*ps, len)); an empty
  sequence gives out = 0 and lse = -inf; query head h reads kv head h // G.
"""
from __future__ import annotations

import numpy as np

TOKEN_MAJOR = "token_major"
XPACKED = "xpacked"


def _as_f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16 and fp32 values are representable in fp64)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _as_int(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def _index(pool, idx):
    """pool[idx] upcast to float64; the pool may be a torch tensor (any dtype) or numpy."""
    try:
        import torch
        if isinstance(pool, torch.Tensor):
            tidx = tuple(torch.as_tensor(i) if isinstance(i, np.ndarray) else i for i in idx)
            return pool[tidx].detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(pool[idx], dtype=np.float64)


def gather_sequence(key_cache, value_cache, layout: str, block_table_row, n: int,
                    block_size: int):
    """Contiguous K and V, each [num_kv_heads, n, head_dim] float64, of one sequence.

    Token t sits in physical block ``block_table_row[t // block_size]`` at slot
    ``t % block_size`` (PagedAttention V2 page, ``_partition_attn_kernel``, paged K/V
    gather; flash-decode post, per-block loop of the unsplit kernel).
    Token-major pools are [num_blocks, KVH, bs, D]; x-packed K is
    [num_blocks, KVH, D / x, bs, x] with element (t, d) at [blk, h, d // x, t % bs, d % x]
    and x-packed V is [num_blocks, KVH, D, bs] with element (t, d) at [blk, h, d, t % bs].
    Only the sequence's own slots are read (then upcast exactly to float64).
    """
    row = _as_int(block_table_row)
    t = np.arange(n)
    blk = row[t // block_size]
    nblocks = key_cache.shape[0]
    if n and (blk.min() < 0 or blk.max() >= nblocks):
        raise ValueError("block table entry outside the pool for a valid token")
    off = t % block_size
    kvh = key_cache.shape[1]
    if layout == TOKEN_MAJOR:
        d_model = key_cache.shape[3]
        K = np.empty((kvh, n, d_model))
        V = np.empty((kvh, n, d_model))
        for h in range(kvh):
            K[h] = _index(key_cache, (blk, h, off, slice(None)))
            V[h] = _index(value_cache, (blk, h, off, slice(None)))
    elif layout == XPACKED:
        x = key_cache.shape[4]
        d_model = key_cache.shape[2] * x
        d = np.arange(d_model)
        K = np.empty((kvh, n, d_model))
        V = np.empty((kvh, n, d_model))
        for h in range(kvh):
            K[h] = _index(key_cache, (blk[:, None], h, (d // x)[None, :], off[:, None], (d % x)[None, :]))
            V[h] = _index(value_cache, (blk[:, None], h, d[None, :], off[:, None]))
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return K, V


def _dequant(x: np.ndarray, cache_scale: float) -> np.ndarray:
    """Values of a quantized cache: the stored value (already upcast exactly to float64)
    times the cache's scale. The PagedAttention V2 page's launcher takes kv_cache_dtype,
    k_scale and v_scale without defining them; the plainest reading is a per-tensor
    dequantization factor, 1 for an unquantized cache."""
    return x * float(cache_scale)


def _kv_head(h: int, group: int) -> int:
    """Query head h belongs to the contiguous group of kv head h // G (both decode pages)."""
    return h // group


def _scores(q_vec: np.ndarray, K: np.ndarray, scale: float, slope=None) -> np.ndarray:
    """s_t = scale * <q, k_t> for every token t of the sequence, plus the ALiBi bias when a
    slope is given.

    ALiBi (Press, Smith and Lewis, "Train Short, Test Long: Attention with Linear Biases
    Enables Input Length Extrapolation", ICLR 2022) adds -m_h * (i - j) to the score of
    query position i on key position j, with a fixed slope m_h per head. The decoded token
    is the sequence's last position, i = n - 1, so key t gets -m_h * (n - 1 - t): zero for
    the token itself and more negative the older the key. (The PagedAttention V2 page's
    launcher takes alibi_slopes but never defines or uses them; this is the published
    definition.)
    """
    s = scale * (K @ q_vec)
    if slope is not None:
        n = K.shape[0]
        s = s - float(slope) * ((n - 1) - np.arange(n))
    return s


def decode(query, key_cache, value_cache, layout: str, block_tables, seq_lens, scale: float,
           num_kv_heads: int, block_size: int, alibi_slopes=None, k_scale: float = 1.0,
           v_scale: float = 1.0):
    """Unsplit decode attention. Returns (out [S,H,D], lse [S,H]) in float64.

    out[b,h] = sum_t softmax(s)_t v_t and lse[b,h] = log sum_t exp(s_t), natural log,
    over the sequence's len_b tokens (with the ALiBi bias of head h when alibi_slopes [H]
    is given). len_b = 0 gives zeros and -inf. A quantized cache (float8 pools) holds
    k_t / k_scale and v_t / v_scale: the keys and values used are the stored values times
    k_scale and v_scale (see _dequant).
    """
    slopes = None if alibi_slopes is None else _as_f64(alibi_slopes)
    q = _as_f64(query)
    bt = _as_int(block_tables)
    lens = _as_int(seq_lens)
    S, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // num_kv_heads
    out = np.zeros((S, H, D))
    lse = np.full((S, H), -np.inf)
    for b in range(S):
        n = int(lens[b])
        if n == 0:
            continue
        K, V = gather_sequence(key_cache, value_cache, layout, bt[b], n, block_size)
        K, V = _dequant(K, k_scale), _dequant(V, v_scale)
        for h in range(H):
            kh = _kv_head(h, G)
            s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[h])
            M = s.max()
            e = np.exp(s - M)
            Z = e.sum()
            out[b, h] = (e @ V[kh]) / Z
            lse[b, h] = M + np.log(Z)
    return out, lse


def partition_ranges(n: int, block_size: int, partition_size: int, num_splits: int = 0):
    """Token ranges [t0, t1) of the non-empty partitions of one n-token sequence.

    Fixed partitions (num_splits = 0; PagedAttention V2 page, ``_partition_attn_kernel``):
    partition p covers [p*ps, min((p+1)*ps, n)) for p < ceil(n / ps).

    NUM_SPLITS policy (num_splits = NS > 0; flash-decode post,
    ``_flash_decode_partial_kernel``): the sequence's nb = ceil(n / bs) pages are cut
    into runs of bps = ceil(nb / NS) whole pages, so split s covers pages
    [s*bps, min((s+1)*bps, nb)), i.e. tokens [s*bps*bs, min((s+1)*bps*bs, n)). Splits
    that start at or past page nb are empty (only ceil(nb / bps) <= NS are real).
    An empty sequence has no partitions.
    """
    if n <= 0:
        return []
    if num_splits > 0:
        nb = -(-n // block_size)
        bps = -(-nb // num_splits)
        span = bps * block_size
    else:
        span = partition_size
    count = -(-n // span)
    return [(p * span, min((p + 1) * span, n)) for p in range(count)]


def decode_partials(query, key_cache, value_cache, layout: str, block_tables, seq_lens,
                    scale: float, num_kv_heads: int, block_size: int, partition_size: int,
                    max_num_partitions: int, num_splits: int = 0, normalized: bool = False,
                    alibi_slopes=None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Split-K partials per (b, h, p): (acc [S,H,P,D], m [S,H,P], l [S,H,P]) in float64.

    Partition p of sequence b covers the token range ``partition_ranges`` gives (fixed
    ps-token partitions, or the NUM_SPLITS page-aligned policy when num_splits > 0). For
    each non-empty one, m = max_t s_t, l = sum_t exp(s_t - m) and
    acc = sum_t exp(s_t - m) v_t (unnormalized, as the flash-decode post's partial kernel
    keeps it), or acc / l when ``normalized`` (the PagedAttention V2 page's tmp_output,
    with l its exp_sums and m its max_logits). Partitions past the sequence's last one
    carry the sentinel m = -inf, l = 0 (PagedAttention V2 page, unused-partition branch);
    their acc is left 0 here and is not part of the contract. With alibi_slopes [H] every
    score carries the ALiBi bias of its absolute position in the sequence (see _scores).
    """
    slopes = None if alibi_slopes is None else _as_f64(alibi_slopes)
    q = _as_f64(query)
    bt = _as_int(block_tables)
    lens = _as_int(seq_lens)
    S, H, D = q.shape
    G = H // num_kv_heads
    P = int(max_num_partitions)
    ps = int(partition_size)
    if ps < 1 and num_splits <= 0:
        raise ValueError("partition_size must be >= 1")
    acc = np.zeros((S, H, P, D))
    m = np.full((S, H, P), -np.inf)
    l = np.zeros((S, H, P))
    for b in range(S):
        n = int(lens[b])
        ranges = partition_ranges(n, block_size, ps, num_splits)
        if not ranges:
            continue
        if len(ranges) > P:
            raise ValueError("max_num_partitions too small for this sequence")
        K, V = gather_sequence(key_cache, value_cache, layout, bt[b], n, block_size)
        K, V = _dequant(K, k_scale), _dequant(V, v_scale)
        for h in range(H):
            kh = _kv_head(h, G)
            s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[h])
            for p, (t0, t1) in enumerate(ranges):
                sp = s[t0:t1]
                mp = sp.max()
                e = np.exp(sp - mp)
                m[b, h, p] = mp
                l[b, h, p] = e.sum()
                acc[b, h, p] = e @ V[kh][t0:t1]
                if normalized:
                    acc[b, h, p] = acc[b, h, p] / l[b, h, p]
    return acc, m, l


def reduce_partials(partial_acc, partial_m, partial_l, seq_lens, partition_size: int,
                    num_splits: int = 0, block_size: int = 16, normalized: bool = False):
    """Cross-partition combine. Returns (out [S,H,D], lse [S,H]) in float64.

    Over the P_b non-empty partitions of sequence b (``partition_ranges``; for fixed
    partitions P_b = ceil(len_b / ps) as in the PagedAttention V2 page's reduce kernel):
    M = max_p m_p, w_p = exp(m_p - M), out = sum_p w_p acc_p / sum_p w_p l_p and
    lse = M + log(sum_p w_p l_p) (flash-decode post, combine kernel). With
    ``normalized`` partials (acc_p already divided by l_p) every partition weighs
    w_p l_p instead: out = sum_p w_p l_p acc_p / sum_p w_p l_p (PagedAttention V2 page,
    ``_reduce_partitions_kernel``). Partitions p >= P_b are never read. len_b = 0 gives
    zeros and -inf.
    """
    acc = _as_f64(partial_acc)
    m = _as_f64(partial_m)
    l = _as_f64(partial_l)
    lens = _as_int(seq_lens)
    S, H, P, D = acc.shape
    out = np.zeros((S, H, D))
    lse = np.full((S, H), -np.inf)
    for b in range(S):
        n = int(lens[b])
        nparts = len(partition_ranges(n, block_size, int(partition_size), num_splits))
        if nparts == 0:
            continue
        for h in range(H):
            mp = m[b, h, :nparts]
            M = mp.max()
            w = np.exp(mp - M)
            Z = w @ l[b, h, :nparts]
            if normalized:
                out[b, h] = ((w * l[b, h, :nparts]) @ acc[b, h, :nparts]) / Z
            else:
                out[b, h] = (w @ acc[b, h, :nparts]) / Z
            lse[b, h] = M + np.log(Z)
    return out, lse
