"""Paged-KV attention for AMD Instinct MI355X (gfx950): Python binding of libpkv.so.

This module only marshals arguments: it checks devices, dtypes, shapes and contiguity
of torch tensors, then passes raw device pointers, sizes and the current HIP stream to
the C ABI declared in ``include/pkv.h``. Every step of the computation runs in the HIP
kernels of ``libpkv.so``; there is no fallback. If the library is missing, every entry
point raises.

Entry points (same names as the C ABI):
  paged_decode_partial(...)   split-K partials (acc, m, l) per (seq, head, partition)
  paged_decode_reduce(...)    LSE-weighted combine of the partials
  paged_decode_split_partial(...), paged_decode_split_reduce(...)
                              the same with NUM_SPLITS page-aligned splits per sequence
  paged_decode(...)           the whole decode: allocates the scratch it needs and runs the
                              one-launch C entry point (or, with one_launch=False, the two
                              phases)
  paged_attention_v2(...)     the PagedAttention V2 launcher (x-packed cache, 512-token
                              partitions, normalized tmp_output / exp_sums / max_logits)
  mla_paged_prefill(...)      MLA causal paged prefill, base-2 LSE (page_size 1, or pages of
                              several tokens through mla_paged_prefill_pages)
  mla_paged_decode(...)       MLA decode (one new token per sequence), split-K
read_bandwidth(...) is a measurement helper (a plain streaming read of a buffer), not part
of the attention path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["mla_decode_default_split", "paged_decode_partial", "paged_decode_reduce", "paged_decode_split_partial",
           "paged_decode_split_reduce", "paged_decode", "paged_decode_into", "paged_decode_static",
           "paged_decode_partial_ex", "paged_decode_ex",
           "paged_attention_v2",
           "mla_paged_prefill", "mla_paged_prefill_pages", "mla_paged_decode", "read_bandwidth", "lib", "library_path", "PkvError", "TOKEN_MAJOR",
           "XPACKED", "num_partitions"]

TOKEN_MAJOR = "token_major"
XPACKED = "xpacked"
_LAYOUT = {TOKEN_MAJOR: 0, XPACKED: 1}
_DTYPE = {torch.float32: 0, torch.bfloat16: 1}

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpkv.so"
_lib = None


class PkvError(RuntimeError):
    """HIP runtime failure reported by the library (status PKV_EHIP)."""


def library_path() -> str:
    """In-tree libpkv.so, or the file named by PKV_LIBRARY (for comparing builds)."""
    return os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """Load libpkv.so (built in-tree by ``python -m paged_kv_gqa_table_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_gqa_table_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.paged_decode_partial.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                       f32, i32, i32, i32, vp, vp, vp, vp]
    L.paged_decode_partial.restype = i32
    L.paged_decode_reduce.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, vp]
    L.paged_decode_reduce.restype = i32
    L.paged_decode_split_partial.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                             f32, i32, i32, vp, vp, vp, vp]
    L.paged_decode_split_partial.restype = i32
    L.paged_decode_split_reduce.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, vp]
    L.paged_decode_split_reduce.restype = i32
    L.paged_decode.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                               i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.paged_decode.restype = i32
    L.paged_attention_v2.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, vp, i32, i32, i32, i32,
                                     i32, i32, i32, vp, i32, f32, f32, vp]
    L.paged_attention_v2.restype = i32
    L.mla_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                    f32, vp, vp, vp]
    L.mla_paged_prefill.restype = i32
    L.mla_paged_prefill_pages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                          i32, f32, vp, vp, vp, vp, vp]
    L.mla_paged_prefill_pages.restype = i32
    L.mla_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                   vp, vp, vp, vp, vp, vp, vp]
    L.mla_paged_decode.restype = i32
    L.paged_decode_partial_ex.argtypes = [vp, i32, vp, vp, i32, i32, f32, f32, vp, vp, i32, vp, i32, i32, i32, i32,
                                          i32, i32, f32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.paged_decode_partial_ex.restype = i32
    L.paged_decode_ex.argtypes = [vp, i32, vp, vp, i32, i32, f32, f32, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                  f32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.paged_decode_ex.restype = i32
    L.paged_decode_static.argtypes = [vp, i32, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                      i32, i32, vp, vp, vp]
    L.paged_decode_static.restype = i32
    L.pkv_read_bandwidth.argtypes = [vp, ctypes.c_size_t, vp, vp]
    L.pkv_read_bandwidth.restype = i32
    L.pkv_last_error.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_version.argtypes = []
    L.pkv_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status == PKV_OK:
        return
    msg = lib().pkv_last_error().decode(errors="replace")
    if status == PKV_EINVAL:
        raise ValueError(f"{what}: {msg}")
    if status == PKV_EUNSUPPORTED:
        raise NotImplementedError(f"{what}: {msg}")
    raise PkvError(f"{what}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(name: str, t: torch.Tensor, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def num_partitions(max_seq_len: int, partition_size: int) -> int:
    return max(1, -(-int(max_seq_len) // int(partition_size)))


def _pool_geometry(key_cache: torch.Tensor, layout: str) -> Tuple[int, int, int]:
    """(num_blocks, block_size, head_dim) of a K pool."""
    if layout == TOKEN_MAJOR:
        if key_cache.dim() != 4:
            raise ValueError("token-major key_cache must be [num_blocks, kv_heads, block_size, head_dim]")
        return key_cache.shape[0], key_cache.shape[2], key_cache.shape[3]
    if layout == XPACKED:
        if key_cache.dim() != 5:
            raise ValueError("x-packed key_cache must be [num_blocks, kv_heads, head_dim/x, block_size, x]")
        return key_cache.shape[0], key_cache.shape[3], key_cache.shape[2] * key_cache.shape[4]
    raise ValueError(f"unknown layout {layout!r}")


def _check_decode_inputs(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads, layout,
                         kv_dtype=None):
    """Common checks of the decode inputs; returns (S, H, D, num_blocks, block_size). The
    caches hold the query's dtype, or ``kv_dtype`` when given (torch.float8_e4m3fn)."""
    if query.dtype not in _DTYPE:
        raise ValueError(f"query dtype {query.dtype} not supported")
    _dev("query", query, ndim=3)
    _dev("key_cache", key_cache, kv_dtype or query.dtype)
    _dev("value_cache", value_cache, kv_dtype or query.dtype)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    S, H, D = query.shape
    nb, bs, kd = _pool_geometry(key_cache, layout)
    if kd != D:
        raise ValueError(f"key_cache head_dim {kd} != query head_dim {D}")
    if key_cache.shape[1] != num_kv_heads or value_cache.shape[1] != num_kv_heads:
        raise ValueError("kv cache head axis does not match num_kv_heads")
    if layout == XPACKED:
        if key_cache.shape[4] != 16 // key_cache.element_size():
            raise ValueError("x-packed key_cache needs x = 16 / element size in its last axis")
        v_shape = (nb, num_kv_heads, D, bs)
    else:
        v_shape = (nb, num_kv_heads, bs, D)
    if tuple(value_cache.shape) != v_shape:
        raise ValueError(f"value_cache must be {v_shape}, got {tuple(value_cache.shape)}")
    if seq_lens.shape[0] != S or block_tables.shape[0] != S:
        raise ValueError("seq_lens / block_tables do not match the batch")
    return S, H, D, nb, bs


def _check_partials(partial_acc, partial_m, partial_l, S, H, D):
    _dev("partial_acc", partial_acc, torch.float32, 4)
    _dev("partial_m", partial_m, torch.float32, 3)
    _dev("partial_l", partial_l, torch.float32, 3)
    P = partial_m.shape[2]
    if tuple(partial_acc.shape) != (S, H, P, D) or tuple(partial_m.shape) != (S, H, P) \
            or tuple(partial_l.shape) != (S, H, P):
        raise ValueError("partials must be [S, H, P, D] and [S, H, P]")
    return P


def _cache_options(query, kv_cache_dtype, k_scale, v_scale, alibi_slopes):
    """(kv dtype code for the C ABI, torch dtype of the caches) for the cache options, or
    (None, None) when they are all at their defaults (an unquantized cache, no ALiBi)."""
    if alibi_slopes is not None:
        _dev("alibi_slopes", alibi_slopes, torch.float32, 1)
        if alibi_slopes.numel() != query.shape[1]:
            raise ValueError("alibi_slopes must hold one slope per query head")
    if kv_cache_dtype in ("fp8", "fp8_e4m3"):
        return 2, torch.float8_e4m3fn
    if kv_cache_dtype != "auto":
        raise NotImplementedError(f"kv_cache_dtype {kv_cache_dtype!r}")
    if float(k_scale) != 1.0 or float(v_scale) != 1.0:
        raise ValueError("k_scale / v_scale apply to a float8 cache only")
    if alibi_slopes is None:
        return None, None
    return _DTYPE[query.dtype], None


def paged_decode_partial(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                         block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                         num_kv_heads: int, partition_size: int, max_seq_len: int,
                         partial_acc: torch.Tensor, partial_m: torch.Tensor, partial_l: torch.Tensor,
                         layout: str = TOKEN_MAJOR, kv_cache_dtype: str = "auto", k_scale: float = 1.0,
                         v_scale: float = 1.0, alibi_slopes: Optional[torch.Tensor] = None) -> None:
    """Phase 1 of split-K decode into caller-allocated partials (asynchronous).

    Cache options (the C paged_decode_partial_ex): ``kv_cache_dtype`` "fp8" / "fp8_e4m3"
    for torch.float8_e4m3fn caches, whose keys and values are k_scale and v_scale times the
    stored values; ``alibi_slopes`` [H] float32 adds the ALiBi bias -slope_h (len - 1 - t)."""
    kv_code, kv_dtype = _cache_options(query, kv_cache_dtype, k_scale, v_scale, alibi_slopes)
    S, H, D, nb, bs = _check_decode_inputs(query, key_cache, value_cache, block_tables, seq_lens,
                                           num_kv_heads, layout, kv_dtype)
    P = _check_partials(partial_acc, partial_m, partial_l, S, H, D)
    if kv_code is not None:
        st = lib().paged_decode_partial_ex(
            _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout], kv_code,
            float(k_scale), float(v_scale), _ptr(alibi_slopes), _ptr(block_tables), block_tables.shape[1],
            _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb, float(scale), int(partition_size), 0, P,
            int(max_seq_len), _ptr(partial_acc), _ptr(partial_m), _ptr(partial_l), _stream(query.device))
        _check(st, "paged_decode_partial_ex")
        return
    st = lib().paged_decode_partial(
        _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout],
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb,
        float(scale), int(partition_size), P, int(max_seq_len), _ptr(partial_acc), _ptr(partial_m),
        _ptr(partial_l), _stream(query.device))
    _check(st, "paged_decode_partial")


def paged_decode_split_partial(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                               block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                               num_kv_heads: int, max_seq_len: int, partial_acc: torch.Tensor,
                               partial_m: torch.Tensor, partial_l: torch.Tensor,
                               layout: str = TOKEN_MAJOR, kv_cache_dtype: str = "auto", k_scale: float = 1.0,
                               v_scale: float = 1.0, alibi_slopes: Optional[torch.Tensor] = None) -> None:
    """Phase 1 with NUM_SPLITS page-aligned splits per sequence; num_splits is the partition
    axis of the partials (asynchronous). Cache options as in paged_decode_partial."""
    kv_code, kv_dtype = _cache_options(query, kv_cache_dtype, k_scale, v_scale, alibi_slopes)
    S, H, D, nb, bs = _check_decode_inputs(query, key_cache, value_cache, block_tables, seq_lens,
                                           num_kv_heads, layout, kv_dtype)
    ns = _check_partials(partial_acc, partial_m, partial_l, S, H, D)
    if kv_code is not None:
        st = lib().paged_decode_partial_ex(
            _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout], kv_code,
            float(k_scale), float(v_scale), _ptr(alibi_slopes), _ptr(block_tables), block_tables.shape[1],
            _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb, float(scale), 0, ns, ns, int(max_seq_len),
            _ptr(partial_acc), _ptr(partial_m), _ptr(partial_l), _stream(query.device))
        _check(st, "paged_decode_partial_ex")
        return
    st = lib().paged_decode_split_partial(
        _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout],
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb,
        float(scale), ns, int(max_seq_len), _ptr(partial_acc), _ptr(partial_m), _ptr(partial_l),
        _stream(query.device))
    _check(st, "paged_decode_split_partial")


def paged_decode_reduce(partial_acc: torch.Tensor, partial_m: torch.Tensor, partial_l: torch.Tensor,
                        seq_lens: torch.Tensor, partition_size: int, out: torch.Tensor,
                        lse: Optional[torch.Tensor] = None) -> None:
    """Phase 2 of split-K decode into caller-allocated out (and lse) (asynchronous)."""
    _dev("partial_acc", partial_acc, torch.float32, 4)
    _dev("partial_m", partial_m, torch.float32, 3)
    _dev("partial_l", partial_l, torch.float32, 3)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    if out.dtype not in _DTYPE:
        raise ValueError(f"out dtype {out.dtype} not supported")
    _dev("out", out, ndim=3)
    S, H, P, D = partial_acc.shape
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [S, H, D]")
    if lse is not None:
        _dev("lse", lse, torch.float32, 2)
        if tuple(lse.shape) != (S, H):
            raise ValueError("lse must be [S, H]")
    st = lib().paged_decode_reduce(_ptr(partial_acc), _ptr(partial_m), _ptr(partial_l), _ptr(seq_lens),
                                   S, H, D, int(partition_size), P, _ptr(out), _DTYPE[out.dtype],
                                   _ptr(lse), _stream(out.device))
    _check(st, "paged_decode_reduce")


def paged_decode_split_reduce(partial_acc: torch.Tensor, partial_m: torch.Tensor, partial_l: torch.Tensor,
                              seq_lens: torch.Tensor, block_size: int, out: torch.Tensor,
                              lse: Optional[torch.Tensor] = None) -> None:
    """Phase 2 for NUM_SPLITS partials (num_splits = their partition axis) (asynchronous)."""
    _dev("partial_acc", partial_acc, torch.float32, 4)
    _dev("partial_m", partial_m, torch.float32, 3)
    _dev("partial_l", partial_l, torch.float32, 3)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    if out.dtype not in _DTYPE:
        raise ValueError(f"out dtype {out.dtype} not supported")
    _dev("out", out, ndim=3)
    S, H, P, D = partial_acc.shape
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [S, H, D]")
    if lse is not None:
        _dev("lse", lse, torch.float32, 2)
        if tuple(lse.shape) != (S, H):
            raise ValueError("lse must be [S, H]")
    st = lib().paged_decode_split_reduce(_ptr(partial_acc), _ptr(partial_m), _ptr(partial_l), _ptr(seq_lens),
                                         S, H, D, int(block_size), P, _ptr(out), _DTYPE[out.dtype], _ptr(lse),
                                         _stream(out.device))
    _check(st, "paged_decode_split_reduce")


def paged_decode_into(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, num_kv_heads: int,
                      partition_size: int, num_splits: int, max_seq_len: int, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, partial_acc: Optional[torch.Tensor] = None,
                      partial_m: Optional[torch.Tensor] = None, partial_l: Optional[torch.Tensor] = None,
                      counters: Optional[torch.Tensor] = None, layout: str = TOKEN_MAJOR,
                      kv_cache_dtype: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0,
                      alibi_slopes: Optional[torch.Tensor] = None) -> None:
    """The one-launch C ``paged_decode`` into caller-allocated buffers (asynchronous).

    With partials of one partition (or none) it is the single pass; otherwise ``counters``
    ([S * num_kv_heads] int32) must be zero and is left zero. Cache options as in
    paged_decode_partial (the C paged_decode_ex)."""
    kv_code, kv_dtype = _cache_options(query, kv_cache_dtype, k_scale, v_scale, alibi_slopes)
    S, H, D, nb, bs = _check_decode_inputs(query, key_cache, value_cache, block_tables, seq_lens,
                                           num_kv_heads, layout, kv_dtype)
    _dev("out", out, query.dtype, 3)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [S, H, D]")
    if lse is not None:
        _dev("lse", lse, torch.float32, 2)
        if tuple(lse.shape) != (S, H):
            raise ValueError("lse must be [S, H]")
    if partial_m is None:
        P = 1
    else:
        P = _check_partials(partial_acc, partial_m, partial_l, S, H, D)
    if counters is not None:
        _dev("counters", counters, torch.int32, 1)
        if counters.numel() < S * num_kv_heads:
            raise ValueError("counters must hold num_seqs * num_kv_heads int32")
    if kv_code is not None:
        st = lib().paged_decode_ex(
            _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout], kv_code,
            float(k_scale), float(v_scale), _ptr(alibi_slopes), _ptr(block_tables), block_tables.shape[1],
            _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb, float(scale), int(partition_size), int(num_splits), P,
            int(max_seq_len), _ptr(partial_acc), _ptr(partial_m), _ptr(partial_l), _ptr(counters), _ptr(out),
            _ptr(lse), _stream(query.device))
        _check(st, "paged_decode_ex")
        return
    st = lib().paged_decode(
        _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout],
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb,
        float(scale), int(partition_size), int(num_splits), P, int(max_seq_len), _ptr(partial_acc),
        _ptr(partial_m), _ptr(partial_l), _ptr(counters), _ptr(out), _ptr(lse), _stream(query.device))
    _check(st, "paged_decode")


def paged_decode_static(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                        block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, num_kv_heads: int,
                        max_seq_len: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                        partition_size: int = 512, num_splits: int = 0, layout: str = TOKEN_MAJOR) -> None:
    """The C ``paged_decode_static`` into caller buffers (asynchronous): the decode with its
    partials in the library's static device scratch, so nothing is allocated (neither here
    nor in the library) and nothing is read back to the host. Calls that overlap in time on
    one GPU race on that scratch."""
    S, H, D, nb, bs = _check_decode_inputs(query, key_cache, value_cache, block_tables, seq_lens,
                                           num_kv_heads, layout)
    _dev("out", out, query.dtype, 3)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [S, H, D]")
    if lse is not None:
        _dev("lse", lse, torch.float32, 2)
        if tuple(lse.shape) != (S, H):
            raise ValueError("lse must be [S, H]")
    st = lib().paged_decode_static(
        _ptr(query), _DTYPE[query.dtype], _ptr(key_cache), _ptr(value_cache), _LAYOUT[layout],
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, H, num_kv_heads, D, bs, nb,
        float(scale), int(partition_size), int(num_splits), int(max_seq_len), _ptr(out), _ptr(lse),
        _stream(query.device))
    _check(st, "paged_decode_static")


def paged_decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                 block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, num_kv_heads: int,
                 partition_size: int = 512, layout: str = TOKEN_MAJOR,
                 max_seq_len: Optional[int] = None, return_lse: bool = False,
                 max_num_partitions: Optional[int] = None, num_splits: int = 0,
                 one_launch: Optional[bool] = None, kv_cache_dtype: str = "auto", k_scale: float = 1.0,
                 v_scale: float = 1.0, alibi_slopes: Optional[torch.Tensor] = None):
    """Decode attention for one new token per sequence; returns ``out`` [S, H, D] in the
    query dtype, or ``(out, lse)``.

    Partitions are ``partition_size`` tokens, or ``num_splits`` page-aligned splits per
    sequence when num_splits > 0. ``one_launch`` runs the C ``paged_decode`` (one kernel;
    partials and zeroed counters are allocated here as its scratch); otherwise the two
    phases run as separate launches. By default (None) one launch is used only when every
    sequence fits one partition (the single pass): with several partitions the launch's
    cross-workgroup combine costs more on MI355X than the second launch it saves.
    ``max_seq_len`` defaults to ``seq_lens.max()`` (one device-to-host read). Cache options
    (float8 caches with their scales, ALiBi slopes) as in paged_decode_partial.
    """
    opts = dict(kv_cache_dtype=kv_cache_dtype, k_scale=k_scale, v_scale=v_scale, alibi_slopes=alibi_slopes)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    S, H, D = query.shape
    if num_splits > 0:
        P = max(int(num_splits), int(max_num_partitions or 0))
    else:
        P = max_num_partitions or num_partitions(max_seq_len, partition_size)
    if one_launch is None:
        one_launch = P == 1
    dev = query.device
    out = torch.empty((S, H, D), dtype=query.dtype, device=dev)
    lse = torch.empty((S, H), dtype=torch.float32, device=dev) if return_lse else None
    acc = m = l = counters = None
    if P > 1 or not one_launch:
        acc = torch.empty((S, H, P, D), dtype=torch.float32, device=dev)
        m = torch.empty((S, H, P), dtype=torch.float32, device=dev)
        l = torch.empty((S, H, P), dtype=torch.float32, device=dev)
    if one_launch:
        if P > 1:
            counters = torch.zeros((S * num_kv_heads,), dtype=torch.int32, device=dev)
        paged_decode_into(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads,
                          partition_size, num_splits, max_seq_len, out, lse, acc, m, l, counters, layout, **opts)
    elif num_splits > 0:
        paged_decode_split_partial(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads,
                                   max_seq_len, acc, m, l, layout=layout, **opts)
        paged_decode_split_reduce(acc, m, l, seq_lens, _pool_geometry(key_cache, layout)[1], out, lse)
    else:
        paged_decode_partial(query, key_cache, value_cache, block_tables, seq_lens, scale, num_kv_heads,
                             partition_size, max_seq_len, acc, m, l, layout=layout, **opts)
        paged_decode_reduce(acc, m, l, seq_lens, partition_size, out, lse)
    return (out, lse) if return_lse else out


def paged_attention_v2(out: torch.Tensor, exp_sums: torch.Tensor, max_logits: torch.Tensor,
                       tmp_output: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, num_kv_heads: int, scale: float,
                       block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                       max_seq_len: int, alibi_slopes: Optional[torch.Tensor] = None,
                       kv_cache_dtype: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0,
                       **kwargs) -> None:
    """The PagedAttention V2 launcher's call, argument for argument (asynchronous).

    x-packed caches, 512-token partitions; tmp_output holds each partition's normalized
    average, exp_sums its l and max_logits its m. ``alibi_slopes`` [H] float32 adds the
    ALiBi bias -slope_h * (len - 1 - t). ``kv_cache_dtype`` "fp8" / "fp8_e4m3": the caches
    are torch.float8_e4m3fn (x-packed with x = 16) and the keys and values used are k_scale
    and v_scale times the stored values.
    """
    if alibi_slopes is not None:
        _dev("alibi_slopes", alibi_slopes, torch.float32, 1)
        if alibi_slopes.numel() != query.shape[1]:
            raise ValueError("alibi_slopes must hold one slope per query head")
    if kv_cache_dtype in ("fp8", "fp8_e4m3"):
        kv_code = 2
        if key_cache.dtype != torch.float8_e4m3fn or value_cache.dtype != torch.float8_e4m3fn:
            raise ValueError("kv_cache_dtype='fp8' needs torch.float8_e4m3fn caches")
        # geometry checks on byte views (same shapes, one byte per element)
        kc_chk, vc_chk = key_cache.view(torch.uint8), value_cache.view(torch.uint8)
    elif kv_cache_dtype == "auto":
        if float(k_scale) != 1.0 or float(v_scale) != 1.0:
            raise ValueError("k_scale / v_scale apply to a float8 cache only")
        kv_code = None
        kc_chk, vc_chk = key_cache, value_cache
    else:
        raise NotImplementedError(f"paged_attention_v2: kv_cache_dtype {kv_cache_dtype!r}")
    if query.dtype not in _DTYPE:
        raise ValueError(f"query dtype {query.dtype} not supported")
    _dev("query", query, ndim=3)
    _dev("key_cache", key_cache)
    _dev("value_cache", value_cache)
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    S, H, D = query.shape
    nb, bs, kd = _pool_geometry(kc_chk, XPACKED)
    x_expect = 16 // key_cache.element_size()
    if kd != D or kc_chk.shape[4] != x_expect or kc_chk.shape[1] != num_kv_heads:
        raise ValueError("key_cache must be [num_blocks, num_kv_heads, head_size / x, block_size, x]")
    if tuple(vc_chk.shape) != (nb, num_kv_heads, D, bs):
        raise ValueError("value_cache must be [num_blocks, num_kv_heads, head_size, block_size]")
    if kv_code is None:
        if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
            raise ValueError("caches must have the query's dtype")
        kv_code = _DTYPE[query.dtype]
    if bs != int(block_size):
        raise ValueError(f"block_size {block_size} does not match the cache ({bs})")
    P = _check_partials(tmp_output, max_logits, exp_sums, S, H, D)
    _dev("out", out, query.dtype, 3)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [S, H, D]")
    st = lib().paged_attention_v2(
        _ptr(out), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_output), _ptr(query), _DTYPE[query.dtype],
        _ptr(key_cache), _ptr(value_cache), int(num_kv_heads), float(scale), _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), S, H, D, bs, nb, int(max_seq_len), P, _ptr(alibi_slopes),
        kv_code, float(k_scale), float(v_scale), _stream(query.device))
    _check(st, "paged_attention_v2")


def mla_paged_prefill(q_nope: torch.Tensor, q_pe: torch.Tensor, ckv_cache: torch.Tensor,
                      kpe_cache: torch.Tensor, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor,
                      kv_indices: torch.Tensor, sm_scale: float, max_q_len: Optional[int] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      kv_last_page_len: Optional[torch.Tensor] = None):
    """MLA causal paged prefill. Returns (out [total_q, H, ckv] bf16, lse [total_q, H] base 2).

    Same argument order as the page's ``_forward``. ``max_q_len`` defaults to the largest
    q_len in ``qo_indptr`` (one device-to-host read, as the page's host-side batch map).
    Caches of ``[num_pages, page_size, dim]`` with page_size > 1 (or a
    ``kv_last_page_len``) go through ``mla_paged_prefill_pages`` with its index scratch
    allocated here.
    """
    _dev("q_nope", q_nope, torch.bfloat16, 3)
    _dev("q_pe", q_pe, torch.bfloat16, 3)
    _dev("ckv_cache", ckv_cache, torch.bfloat16, 3)
    _dev("kpe_cache", kpe_cache, torch.bfloat16, 3)
    _dev("qo_indptr", qo_indptr, torch.int32, 1)
    _dev("kv_indptr", kv_indptr, torch.int32, 1)
    _dev("kv_indices", kv_indices, torch.int32, 1)
    total_q, H, Dc = q_nope.shape
    Dp = q_pe.shape[2]
    num_pages, page_size, _ = ckv_cache.shape
    if q_pe.shape[:2] != q_nope.shape[:2] or kpe_cache.shape[:2] != ckv_cache.shape[:2] \
            or ckv_cache.shape[2] != Dc or kpe_cache.shape[2] != Dp:
        raise ValueError("inconsistent MLA shapes")
    batch = qo_indptr.shape[0] - 1
    if kv_indptr.shape[0] != batch + 1 or batch < 0:
        raise ValueError("qo_indptr and kv_indptr must both be [batch + 1]")
    if max_q_len is None:
        max_q_len = int((qo_indptr[1:] - qo_indptr[:-1]).max().item()) if batch > 0 else 0
    if out is None:
        out = torch.empty((total_q, H, Dc), dtype=torch.bfloat16, device=q_nope.device)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q_nope.device)
    _dev("out", out, torch.bfloat16, 3)
    _dev("lse", lse, torch.float32, 2)
    if page_size > 1 or kv_last_page_len is not None:
        n_idx = kv_indices.numel()
        tok_indptr = torch.empty((batch + 1,), dtype=torch.int32, device=q_nope.device)
        tok_rows = torch.empty((max(1, n_idx * page_size),), dtype=torch.int32, device=q_nope.device)
        mla_paged_prefill_pages(q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_indptr, kv_indices,
                                kv_last_page_len, sm_scale, int(max_q_len), tok_indptr, tok_rows, out, lse)
        return out, lse
    st = lib().mla_paged_prefill(_ptr(q_nope), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache),
                                 _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices), batch, total_q,
                                 int(max_q_len), num_pages, H, Dc, Dp, page_size, float(sm_scale),
                                 _ptr(out), _ptr(lse), _stream(q_nope.device))
    _check(st, "mla_paged_prefill")
    return out, lse


def mla_paged_prefill_pages(q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_indptr, kv_indices,
                            kv_last_page_len, sm_scale: float, max_q_len: int, token_indptr: torch.Tensor,
                            token_rows: torch.Tensor, out: torch.Tensor, lse: torch.Tensor) -> None:
    """MLA prefill over pages of several tokens into caller buffers (asynchronous);
    token_indptr [batch + 1] and token_rows [num_kv_indices * page_size] int32 are scratch."""
    for n, t in (("q_nope", q_nope), ("q_pe", q_pe), ("ckv_cache", ckv_cache), ("kpe_cache", kpe_cache),
                 ("out", out)):
        _dev(n, t, torch.bfloat16, 3)
    for n, t in (("qo_indptr", qo_indptr), ("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
                 ("token_indptr", token_indptr), ("token_rows", token_rows)):
        _dev(n, t, torch.int32, 1)
    _dev("lse", lse, torch.float32, 2)
    if kv_last_page_len is not None:
        _dev("kv_last_page_len", kv_last_page_len, torch.int32, 1)
    total_q, H, Dc = q_nope.shape
    Dp = q_pe.shape[2]
    num_pages, page_size, _ = ckv_cache.shape
    batch = qo_indptr.shape[0] - 1
    n_idx = kv_indices.numel()
    if token_indptr.numel() < batch + 1 or token_rows.numel() < n_idx * page_size:
        raise ValueError("token_indptr / token_rows scratch too small")
    if kv_last_page_len is not None and kv_last_page_len.numel() < batch:
        raise ValueError("kv_last_page_len must hold one entry per batch")
    st = lib().mla_paged_prefill_pages(
        _ptr(q_nope), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(qo_indptr), _ptr(kv_indptr),
        _ptr(kv_indices), _ptr(kv_last_page_len), batch, total_q, int(max_q_len), num_pages, n_idx, H, Dc, Dp,
        page_size, float(sm_scale), _ptr(token_indptr), _ptr(token_rows), _ptr(out), _ptr(lse),
        _stream(q_nope.device))
    _check(st, "mla_paged_prefill_pages")


def mla_decode_default_split(batch: int, max_kv_len: int, total_keys: int, device=None,
                             kv_lens: Optional[Sequence[int]] = None, cus: Optional[int] = None) -> int:
    """Keys per split for an MLA decode such that every non-empty (split, sequence) item runs
    in one round of one workgroup per compute unit (CU). Two bounds each guarantee that:
    max_kv_len / (CUs // batch) keeps the batch x splits grid within the CUs, and, for
    batches of at most 256 (whose non-empty items the kernel packs onto the lowest workgroup
    ids), total_keys / (CUs - batch) keeps the items, at most total / split + batch, within
    them. With the lengths on the host (``kv_lens``) and at most 256 batches, the split is
    instead the shortest multiple of 16 whose items, sum of ceil(len / split), fit the CUs.
    Otherwise the shorter bound, rounded up to 16 keys. Shorter splits than that lose: each
    split costs a 32 KB partial row and an LDS merge, and a second round waits for the first.
    ``cus`` is the compute-unit count (default: that of ``device``)."""
    if cus is None:
        cus = torch.cuda.get_device_properties(device).multi_processor_count
    cus = int(cus)
    B = max(1, int(batch))
    per_seq = max(1, cus // B)
    split = -(-max(1, int(max_kv_len)) // per_seq)
    if B <= 256 and cus > B and total_keys > 0:
        split = min(split, -(-int(total_keys) // (cus - B)))
    split = max(16, -(-split // 16) * 16)
    if kv_lens is not None and B <= 256 and len(kv_lens) > 0:
        lens = [max(0, int(x)) for x in kv_lens]
        def items(sp):
            return sum(-(-x // sp) for x in lens)
        lo, hi = 1, split // 16  # in units of 16 keys; `split` itself fits (both bounds above)
        if items(hi * 16) <= cus:
            while lo < hi:  # items(s) does not grow with s
                mid = (lo + hi) // 2
                if items(mid * 16) <= cus:
                    hi = mid
                else:
                    lo = mid + 1
            split = hi * 16
    return split


def mla_paged_decode(q_nope: torch.Tensor, q_pe: torch.Tensor, ckv_cache: torch.Tensor, kpe_cache: torch.Tensor,
                     kv_indptr: torch.Tensor, kv_indices: torch.Tensor, sm_scale: float,
                     split_tokens: Optional[int] = None, max_kv_len: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     partials: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                     counters: Optional[torch.Tensor] = None):
    """MLA decode, one new token per sequence: q_nope [B, 16, 512], q_pe [B, 16, 64].
    Returns (out [B, 16, 512] bf16, lse [B, 16] base 2). ``split_tokens`` keys per split,
    by default ``mla_decode_default_split``. Host reads: with both ``split_tokens`` and
    ``max_kv_len`` given nothing is read back (the call stays asynchronous, as a decode loop
    or a captured graph needs: compute the split once and pass it); with ``max_kv_len``
    given and no split, the split comes from the length bounds alone, again without a read;
    with neither, kv_indptr is read to the host once (up to 256 batches the split then fits
    the exact lengths). ``partials`` (acc, m, l) scratch is allocated when not given.
    ``counters``: an int32 [B] device tensor of zeros (left zero by the call) makes it one
    launch, the last workgroup of each batch combining its splits; without it a second
    launch combines."""
    for n, t in (("q_nope", q_nope), ("q_pe", q_pe), ("ckv_cache", ckv_cache), ("kpe_cache", kpe_cache)):
        _dev(n, t, torch.bfloat16, 3)
    _dev("kv_indptr", kv_indptr, torch.int32, 1)
    _dev("kv_indices", kv_indices, torch.int32, 1)
    B, H, Dc = q_nope.shape
    Dp = q_pe.shape[2]
    num_pages, page_size, _ = ckv_cache.shape
    if kv_indptr.numel() != B + 1 or q_pe.shape[:2] != q_nope.shape[:2]:
        raise ValueError("q_nope / q_pe must be [batch, heads, dim] and kv_indptr [batch + 1]")
    host_lens = None
    if max_kv_len is None and B > 0:  # one device-to-host read of the offsets
        ptr = kv_indptr.cpu()
        host_lens = (ptr[1:] - ptr[:-1]).tolist()
        max_kv_len = max(0, max(host_lens))
    if max_kv_len is None:
        max_kv_len = 0
    dev = q_nope.device
    if split_tokens is None:
        split_tokens = mla_decode_default_split(B, int(max_kv_len), kv_indices.numel(), dev, kv_lens=host_lens)
    P = max(1, -(-int(max_kv_len) // int(split_tokens)))
    if partials is None:
        partials = (torch.empty((B, H, P, Dc), dtype=torch.float32, device=dev),
                    torch.empty((B, H, P), dtype=torch.float32, device=dev),
                    torch.empty((B, H, P), dtype=torch.float32, device=dev))
    acc, m, l = partials
    _check_partials(acc, m, l, B, H, Dc)
    if out is None:
        out = torch.empty((B, H, Dc), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _dev("out", out, torch.bfloat16, 3)
    _dev("lse", lse, torch.float32, 2)
    if counters is not None:
        _dev("counters", counters, torch.int32, 1)
        if counters.numel() < B:
            raise ValueError("counters must hold one int32 per batch")
    st = lib().mla_paged_decode(_ptr(q_nope), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(kv_indptr),
                                _ptr(kv_indices), B, num_pages, kv_indices.numel(), int(max_kv_len), H, Dc, Dp,
                                page_size, float(sm_scale), int(split_tokens), m.shape[2], _ptr(acc), _ptr(m),
                                _ptr(l), None if counters is None else _ptr(counters), _ptr(out), _ptr(lse),
                                _stream(dev))
    _check(st, "mla_paged_decode")
    return out, lse


def read_bandwidth(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read all of ``buf`` once on the current stream (plain streaming read; time it with
    events for the read bandwidth). ``sink`` is a 1-element int32 device tensor the kernel
    may write; its value is unspecified."""
    _dev("buf", buf)
    _dev("sink", sink, torch.int32)
    if sink.numel() < 1:
        raise ValueError("sink must hold at least one int32")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().pkv_read_bandwidth(_ptr(buf), nbytes, _ptr(sink), _stream(buf.device)), "pkv_read_bandwidth")
