"""Seeded synthetic workloads for paged-KV decode and MLA paged prefill.

This module only draws random numbers and lays them out (page pools, page
tables, length mixes, layout conversions, NaN canaries). It holds none of the
attention arithmetic, so both the float64 oracle and the HIP path can consume
what it produces without sharing any of the method's code.

Recipe (fixed draw order per case, one ``numpy.random.default_rng(seed)``):
  decode: lengths -> page permutation -> q -> K pool -> V pool
  MLA:    q_len -> prefix -> kv-token permutation -> q_nope -> q_pe -> ckv -> kpe
Values are float32 N(0, 1), cast to the case dtype by torch (round to nearest
even). Integer ranges are inclusive. Every slot of a pool is drawn, including
tail slots past a sequence's length and blocks no sequence owns.

Layouts (names of the pages' own argument comments):
  token-major: K and V are [num_blocks, num_kv_heads, block_size, head_dim]
               (flash-decode blog post, kernel argument comments).
  x-packed:    K is [num_blocks, num_kv_heads, head_dim / x, block_size, x] with
               x = 16 bytes / element size, V is [num_blocks, num_kv_heads,
               head_dim, block_size] (PagedAttention V2 Triton page, kernel
               argument comments).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

TOKEN_MAJOR = "token_major"
XPACKED = "xpacked"

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_ELEM_BYTES = {"f32": 4, "bf16": 2}


def x_pack_factor(dtype: str) -> int:
    """Elements per 16-byte chunk of the x-packed key cache."""
    return 16 // _ELEM_BYTES[dtype]


def elem_bytes(dtype: str) -> int:
    return _ELEM_BYTES[dtype]


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH_DTYPE[dtype])


def token_major_to_xpacked(k_tm: torch.Tensor, v_tm: torch.Tensor):
    """Re-lay a token-major K/V pool in the x-packed layout (pure data movement)."""
    nb, kvh, bs, d = k_tm.shape
    x = 16 // k_tm.element_size()
    k_xp = k_tm.reshape(nb, kvh, bs, d // x, x).permute(0, 1, 3, 2, 4).contiguous()
    v_xp = v_tm.permute(0, 1, 3, 2).contiguous()
    return k_xp, v_xp


def xpacked_to_token_major(k_xp: torch.Tensor, v_xp: torch.Tensor):
    """Inverse of :func:`token_major_to_xpacked`."""
    nb, kvh, dx, bs, x = k_xp.shape
    k_tm = k_xp.permute(0, 1, 3, 2, 4).reshape(nb, kvh, bs, dx * x).contiguous()
    v_tm = v_xp.permute(0, 1, 3, 2).contiguous()
    return k_tm, v_tm


def fp8_pools(case, layout: str) -> tuple:
    """The case's K/V pools cast to float8 e4m3 (torch RNE with the format's range), laid out
    token-major or x-packed with x = 16 (one byte per element)."""
    k, v = case.key_cache, case.value_cache
    if case.layout == XPACKED:
        k, v = xpacked_to_token_major(k, v)
    k8 = k.to(torch.float32).to(torch.float8_e4m3fn)
    v8 = v.to(torch.float32).to(torch.float8_e4m3fn)
    return token_major_to_xpacked(k8, v8) if layout == XPACKED else (k8.contiguous(), v8.contiguous())


def fp8_xpacked_pools(case) -> tuple:
    """The float8 cache the PagedAttention V2 interface reads: x-packed, x = 16."""
    return fp8_pools(case, XPACKED)


@dataclasses.dataclass
class DecodeCase:
    """One batch of single-token decode work over a paged KV cache (CPU tensors)."""

    name: str
    dtype: str                 # "f32" | "bf16"
    layout: str                # TOKEN_MAJOR | XPACKED
    query: torch.Tensor        # [S, H, D]
    key_cache: torch.Tensor    # layout-dependent, see module docstring
    value_cache: torch.Tensor
    block_tables: torch.Tensor  # [S, max_blocks_per_seq] int32, -1 past each sequence
    seq_lens: torch.Tensor     # [S] int32
    num_kv_heads: int
    block_size: int
    scale: float
    partition_size: int

    @property
    def num_seqs(self) -> int:
        return int(self.query.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.query.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.query.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max().item()) if self.num_seqs else 0

    def num_partitions(self, partition_size: Optional[int] = None) -> int:
        ps = partition_size or self.partition_size
        return max(1, -(-self.max_seq_len // ps))

    def kv_bytes(self) -> int:
        """K and V bytes a step must read: sum(len) * KVH * 2 * D * elem."""
        total_tokens = int(self.seq_lens.to(torch.int64).sum().item())
        return total_tokens * self.num_kv_heads * 2 * self.head_dim * elem_bytes(self.dtype)

    def with_layout(self, layout: str) -> "DecodeCase":
        if layout == self.layout:
            return self
        if layout == XPACKED:
            k, v = token_major_to_xpacked(self.key_cache, self.value_cache)
        else:
            k, v = xpacked_to_token_major(self.key_cache, self.value_cache)
        return dataclasses.replace(self, layout=layout, key_cache=k, value_cache=v,
                                   name=f"{self.name}/{layout}")


def _page_tables(rng, lens: np.ndarray, block_size: int, num_blocks: Optional[int],
                 slack: float):
    pages = [-(-int(n) // block_size) for n in lens]
    need = sum(pages)
    if num_blocks is None:
        num_blocks = max(1, math.ceil((1.0 + slack) * need))
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need} pages")
    perm = rng.permutation(num_blocks)
    width = max(1, max(pages) if len(pages) else 1)
    bt = np.full((len(lens), width), -1, dtype=np.int32)
    cur = 0
    for b, nb in enumerate(pages):
        bt[b, :nb] = perm[cur:cur + nb]
        cur += nb
    return bt, num_blocks


def make_decode(lens: Sequence[int], num_heads: int, num_kv_heads: int, head_dim: int,
                dtype: str = "bf16", layout: str = TOKEN_MAJOR, block_size: int = 16,
                seed: int = 0, num_blocks: Optional[int] = None, slack: float = 0.1,
                scale: Optional[float] = None, partition_size: int = 512,
                name: str = "decode", rng=None) -> DecodeCase:
    """Draw one decode batch. ``lens`` may be given or drawn by the caller via ``rng``."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    bt, num_blocks = _page_tables(rng, lens, block_size, num_blocks, slack)
    S = len(lens)
    q = rng.standard_normal((S, num_heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((num_blocks, num_kv_heads, block_size, head_dim), dtype=np.float32)
    k_t = _cast(k, dtype)
    del k
    v = rng.standard_normal((num_blocks, num_kv_heads, block_size, head_dim), dtype=np.float32)
    v_t = _cast(v, dtype)
    del v
    case = DecodeCase(
        name=name, dtype=dtype, layout=TOKEN_MAJOR, query=_cast(q, dtype),
        key_cache=k_t, value_cache=v_t,
        block_tables=torch.from_numpy(bt), seq_lens=torch.from_numpy(lens.astype(np.int32)),
        num_kv_heads=num_kv_heads, block_size=block_size,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
        partition_size=partition_size)
    return case.with_layout(layout)


# --------------------------------------------------------------------------------------
# The five workloads. Each is named by what it is; the index is only the seed.
# --------------------------------------------------------------------------------------

def tiny_fp32(seed: int = 0, partition_size: int = 128) -> DecodeCase:
    """B=2, H=4, KVH=2, D=64, fp32, lens {37, 100}, 16-block pool, scale 1/8."""
    return make_decode([37, 100], 4, 2, 64, dtype="f32", layout=TOKEN_MAJOR, seed=seed,
                       num_blocks=16, scale=1.0 / math.sqrt(64), partition_size=partition_size,
                       name="tiny_fp32_b2_h4_kv2_d64")


def llama_gqa4(seed: int = 1) -> DecodeCase:
    """B=32, H=32, KVH=8, D=128, bf16, lens U[512, 4096], token-major, ps 512."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4096, 32, endpoint=True)
    return make_decode(lens, 32, 8, 128, dtype="bf16", layout=TOKEN_MAJOR, rng=rng,
                       partition_size=512, name="llama_gqa4_b32_h32_kv8_d128")


def wide_gqa6(seed: int = 2, layout: str = XPACKED) -> DecodeCase:
    """B=16, H=24, KVH=4, D=256, bf16, lens U[8192, 32768], x-packed (x=8), ps 512."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(8192, 32768, 16, endpoint=True)
    return make_decode(lens, 24, 4, 256, dtype="bf16", layout=layout, rng=rng,
                       partition_size=512, name="wide_gqa6_b16_h24_kv4_d256")


def skewed_gqa8(seed: int = 3, long_first: bool = True) -> DecodeCase:
    """B=128, H=64, KVH=8, D=128, bf16: one 65536-token sequence + 127 of U[128, 1024]."""
    rng = np.random.default_rng(seed)
    short = rng.integers(128, 1024, 127, endpoint=True)
    lens = np.concatenate([[65536], short]) if long_first else np.concatenate([short, [65536]])
    return make_decode(lens, 64, 8, 128, dtype="bf16", layout=TOKEN_MAJOR, rng=rng,
                       partition_size=512, name="skewed_gqa8_b128_h64_kv8_d128")


def decode_workload(name: str, **kw) -> DecodeCase:
    table = {"tiny_fp32": tiny_fp32, "llama_gqa4": llama_gqa4, "wide_gqa6": wide_gqa6,
             "skewed_gqa8": skewed_gqa8}
    return table[name](**kw)


def with_nan_canaries(case: DecodeCase) -> DecodeCase:
    """Copy of ``case`` whose never-valid KV slots hold NaN.

    NaN goes into every slot a correct kernel must not read: slots past each
    sequence's length inside its last page, and every pool block no sequence owns.
    """
    k = case.key_cache.clone()
    v = case.value_cache.clone()
    bs = case.block_size
    owned = set()
    lens = case.seq_lens.tolist()
    bt = case.block_tables
    for b, n in enumerate(lens):
        nb = -(-n // bs)
        for i in range(nb):
            owned.add(int(bt[b, i]))
        tail = n % bs
        if nb and tail:
            blk = int(bt[b, nb - 1])
            if case.layout == TOKEN_MAJOR:
                k[blk, :, tail:, :] = float("nan")
                v[blk, :, tail:, :] = float("nan")
            else:
                k[blk, :, :, tail:, :] = float("nan")
                v[blk, :, :, tail:] = float("nan")
    unused = [i for i in range(case.num_blocks) if i not in owned]
    if unused:
        idx = torch.tensor(unused, dtype=torch.long)
        k[idx] = float("nan")
        v[idx] = float("nan")
    return dataclasses.replace(case, key_cache=k, value_cache=v, name=case.name + "/nan")


def permute_pool(case: DecodeCase, seed: int) -> DecodeCase:
    """Same logical batch with the pool's block axis permuted and the tables remapped."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(case.num_blocks)        # new block i holds old block perm[i]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(case.num_blocks)
    p = torch.from_numpy(perm).long()
    bt = case.block_tables.clone()
    mask = bt >= 0
    bt[mask] = torch.from_numpy(inv.astype(np.int32))[bt[mask].long()]
    return dataclasses.replace(case, key_cache=case.key_cache[p].contiguous(),
                               value_cache=case.value_cache[p].contiguous(),
                               block_tables=bt, name=case.name + "/perm")


# --------------------------------------------------------------------------------------
# MLA causal paged prefill (page_size 1)
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class MlaCase:
    name: str
    q_nope: torch.Tensor     # [total_q, H, ckv_dim] bf16
    q_pe: torch.Tensor       # [total_q, H, kpe_dim] bf16
    ckv_cache: torch.Tensor  # [num_pages, 1, ckv_dim] bf16
    kpe_cache: torch.Tensor  # [num_pages, 1, kpe_dim] bf16
    qo_indptr: torch.Tensor  # [batch + 1] int32
    kv_indptr: torch.Tensor  # [batch + 1] int32
    kv_indices: torch.Tensor  # [kv_indptr[-1]] int32
    sm_scale: float
    kv_last_page_len: Optional[torch.Tensor] = None  # [batch] int32 when pages hold several tokens

    @property
    def batch(self) -> int:
        return int(self.qo_indptr.numel()) - 1

    @property
    def total_q(self) -> int:
        return int(self.q_nope.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.ckv_cache.shape[0])

    @property
    def page_size(self) -> int:
        return int(self.ckv_cache.shape[1])

    def kv_lens(self) -> List[int]:
        """Key tokens per batch: pages times page size, the last page counted by its length."""
        kv = self.kv_indptr.tolist()
        ps = self.page_size
        last = self.kv_last_page_len.tolist() if self.kv_last_page_len is not None else [ps] * self.batch
        return [((kv[b + 1] - kv[b] - 1) * ps + last[b]) if kv[b + 1] > kv[b] else 0 for b in range(self.batch)]

    @property
    def max_q_len(self) -> int:
        d = (self.qo_indptr[1:] - self.qo_indptr[:-1])
        return int(d.max().item()) if d.numel() else 0

    def visible_pairs(self) -> int:
        """Number of (query token, key token) pairs the causal mask keeps, per head."""
        qo = self.qo_indptr.tolist()
        kvl = self.kv_lens()
        tot = 0
        for b in range(self.batch):
            ql = qo[b + 1] - qo[b]
            kl = kvl[b]
            pre = kl - ql
            tot += sum(pre + i + 1 for i in range(ql))
        return tot


def make_mla(q_lens: Sequence[int], prefixes: Sequence[int], num_heads: int = 16,
             ckv_dim: int = 512, kpe_dim: int = 64, seed: int = 4,
             sm_scale: Optional[float] = None, extra_pages: int = 0, rng=None,
             name: str = "mla") -> MlaCase:
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    prefixes = np.asarray(prefixes, dtype=np.int64)
    kv_lens = prefixes + q_lens
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    num_pages = int(kv[-1]) + extra_pages
    perm = rng.permutation(num_pages)[: int(kv[-1])].astype(np.int32)
    total_q = int(qo[-1])
    q_nope = rng.standard_normal((total_q, num_heads, ckv_dim), dtype=np.float32)
    q_pe = rng.standard_normal((total_q, num_heads, kpe_dim), dtype=np.float32)
    ckv = rng.standard_normal((num_pages, 1, ckv_dim), dtype=np.float32)
    kpe = rng.standard_normal((num_pages, 1, kpe_dim), dtype=np.float32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(192.0)
    return MlaCase(name=name, q_nope=_cast(q_nope, "bf16"), q_pe=_cast(q_pe, "bf16"),
                   ckv_cache=_cast(ckv, "bf16"), kpe_cache=_cast(kpe, "bf16"),
                   qo_indptr=torch.from_numpy(qo), kv_indptr=torch.from_numpy(kv),
                   kv_indices=torch.from_numpy(perm), sm_scale=float(sm_scale))


def make_mla_paged(q_lens: Sequence[int], prefixes: Sequence[int], page_size: int, num_heads: int = 16,
                   ckv_dim: int = 512, kpe_dim: int = 64, seed: int = 4, sm_scale: Optional[float] = None,
                   extra_pages: int = 3, rng=None, name: str = "mla_paged") -> MlaCase:
    """A batch over pages of page_size tokens: batch b gets ceil(kv_len / page_size) pages
    from a random permutation of the pool, its last page holding the remainder
    (kv_last_page_len); every slot of the pool is drawn, unowned slots too.
    Draw order: page permutation -> q_nope -> q_pe -> ckv -> kpe."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(prefixes, dtype=np.int64) + q_lens
    pages_b = (kv_lens + page_size - 1) // page_size
    last = np.where(pages_b > 0, kv_lens - (pages_b - 1) * page_size, page_size).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(pages_b)]).astype(np.int32)
    num_pages = int(kv[-1]) + extra_pages
    perm = rng.permutation(num_pages)[: int(kv[-1])].astype(np.int32)
    total_q = int(qo[-1])
    q_nope = rng.standard_normal((total_q, num_heads, ckv_dim), dtype=np.float32)
    q_pe = rng.standard_normal((total_q, num_heads, kpe_dim), dtype=np.float32)
    ckv = rng.standard_normal((num_pages, page_size, ckv_dim), dtype=np.float32)
    kpe = rng.standard_normal((num_pages, page_size, kpe_dim), dtype=np.float32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(192.0)
    return MlaCase(name=name, q_nope=_cast(q_nope, "bf16"), q_pe=_cast(q_pe, "bf16"),
                   ckv_cache=_cast(ckv, "bf16"), kpe_cache=_cast(kpe, "bf16"),
                   qo_indptr=torch.from_numpy(qo), kv_indptr=torch.from_numpy(kv),
                   kv_indices=torch.from_numpy(perm), sm_scale=float(sm_scale),
                   kv_last_page_len=torch.from_numpy(last))


def mla_prefill_b8(seed: int = 4) -> MlaCase:
    """B=8, 16 heads, ckv 512, kpe 64, page_size 1; q_len U[1,512], prefix U[0,4096]."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, 512, 8, endpoint=True)
    prefixes = rng.integers(0, 4096, 8, endpoint=True)
    return make_mla(q_lens, prefixes, rng=rng, sm_scale=1.0 / math.sqrt(192.0),
                    name="mla_prefill_b8_h16_ckv512_kpe64")


def mla_prefill_b8_pages(page_size: int, seed: int = 4) -> MlaCase:
    """The same batch shapes as mla_prefill_b8 (same q_len and prefix draws) over pages of
    page_size tokens."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, 512, 8, endpoint=True)
    prefixes = rng.integers(0, 4096, 8, endpoint=True)
    return make_mla_paged(q_lens, prefixes, page_size, rng=rng, sm_scale=1.0 / math.sqrt(192.0),
                          name=f"mla_prefill_b8_pages{page_size}")


def mla_decode_b64(seed: int = 6) -> MlaCase:
    """MLA decode shapes: 64 sequences of one new token each (q_len 1) over prefixes
    U[1024, 4096], 16 heads, ckv 512, kpe 64, page_size 1."""
    rng = np.random.default_rng(seed)
    prefixes = rng.integers(1024, 4096, 64, endpoint=True)
    return make_mla(np.ones(64, dtype=np.int64), prefixes, rng=rng, sm_scale=1.0 / math.sqrt(192.0),
                    name="mla_decode_b64_h16_ckv512_kpe64")


def all_decode_names() -> List[str]:
    return ["tiny_fp32", "llama_gqa4", "wide_gqa6", "skewed_gqa8"]
