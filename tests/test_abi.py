"""C-ABI boundary on the host: the library loads, exports what include/pkv.h declares,
and rejects bad arguments with the documented status before any HIP call.

No compute is launched here: every call either fails validation or is a documented
no-op (empty batch), so these tests run without a GPU.
"""
import ctypes
import os
import re

import pytest

import paged_kv_gqa_table_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, EINVAL, EUNSUP = 0, 1, 2
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails (or no-ops) first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pkv.library_path()):
        pytest.skip("libpkv.so not built")
    return pkv.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert {"paged_decode_partial", "paged_decode_reduce", "mla_paged_prefill", "pkv_last_error",
            "pkv_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libpkv.so does not export {n}"


def test_version(L):
    assert L.pkv_version().decode().startswith("pkv ")


def _partial(L, **kw):
    a = dict(query=FAKE, dtype=1, kc=FAKE, vc=FAKE, layout=0, bt=FAKE, mb=8, lens=FAKE, S=2, H=8, KVH=2,
             D=128, bs=16, nb=64, scale=0.1, ps=512, P=1, max_seq_len=128, acc=FAKE, m=FAKE, l=FAKE,
             stream=None)
    a.update(kw)
    return L.paged_decode_partial(a["query"], a["dtype"], a["kc"], a["vc"], a["layout"], a["bt"], a["mb"],
                                  a["lens"], a["S"], a["H"], a["KVH"], a["D"], a["bs"], a["nb"], a["scale"],
                                  a["ps"], a["P"], a["max_seq_len"], a["acc"], a["m"], a["l"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=6, KVH=4), EINVAL),                      # H not a multiple of KVH
    (dict(ps=500), EINVAL),                           # partition not a multiple of block_size
    (dict(ps=0), EINVAL),
    (dict(P=1, max_seq_len=1024), EINVAL),            # too few partitions for max_seq_len
    (dict(mb=4, max_seq_len=65), EINVAL),             # max_seq_len beyond the table width
    (dict(query=None), EINVAL),
    (dict(acc=None), EINVAL),
    (dict(dtype=7), EINVAL),
    (dict(layout=3), EINVAL),
    (dict(S=-1), EINVAL),
    (dict(max_seq_len=-1), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(bs=8, ps=500, mb=64), EINVAL),             # partition size not a multiple of block size 8
    (dict(bs=0), EINVAL),
    (dict(D=96), EUNSUP),
    (dict(H=34, KVH=2), EUNSUP),                      # G = 17
    (dict(S=1 << 20, H=4096, KVH=4096), EUNSUP),      # 2^32 workgroups
    (dict(S=0, query=None), OK),                      # empty batch: nothing to do
    (dict(max_seq_len=0), OK),                        # every sequence empty: nothing touched
])
def test_decode_partial_validation(L, kw, code):
    assert _partial(L, **kw) == code
    if code != OK:
        assert len(L.pkv_last_error()) > 0


def _reduce(L, **kw):
    a = dict(acc=FAKE, m=FAKE, l=FAKE, lens=FAKE, S=2, H=8, D=128, ps=512, P=4, out=FAKE, dt=1, lse=None,
             stream=None)
    a.update(kw)
    return L.paged_decode_reduce(a["acc"], a["m"], a["l"], a["lens"], a["S"], a["H"], a["D"], a["ps"], a["P"],
                                 a["out"], a["dt"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), EINVAL),
    (dict(ps=0), EINVAL),
    (dict(P=0), EINVAL),
    (dict(dt=5), EINVAL),
    (dict(D=0), EINVAL),
    (dict(D=96), EUNSUP),
    (dict(S=0, acc=None), OK),
])
def test_decode_reduce_validation(L, kw, code):
    assert _reduce(L, **kw) == code


def _mla(L, **kw):
    a = dict(qn=FAKE, qp=FAKE, ckv=FAKE, kpe=FAKE, qo=FAKE, kvp=FAKE, idx=FAKE, batch=2, total_q=10,
             max_q_len=6, num_pages=40, H=16, Dc=512, Dp=64, ps=1, sm=0.07, out=FAKE, lse=FAKE, stream=None)
    a.update(kw)
    return L.mla_paged_prefill(a["qn"], a["qp"], a["ckv"], a["kpe"], a["qo"], a["kvp"], a["idx"], a["batch"],
                               a["total_q"], a["max_q_len"], a["num_pages"], a["H"], a["Dc"], a["Dp"], a["ps"],
                               a["sm"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(H=8), EUNSUP),
    (dict(Dc=256), EUNSUP),
    (dict(Dp=32), EUNSUP),
    (dict(ps=16), EUNSUP),
    (dict(out=None), EINVAL),
    (dict(max_q_len=0), EINVAL),
    (dict(batch=-1), EINVAL),
    (dict(sm=float("inf")), EINVAL),
    (dict(total_q=0, qn=None), OK),
])
def test_mla_validation(L, kw, code):
    assert _mla(L, **kw) == code


@pytest.mark.parametrize("buf,nbytes,sink,code", [
    (None, 1024, FAKE, EINVAL),
    (FAKE, 1024, None, EINVAL),
    (FAKE, 1000, FAKE, EINVAL),        # not a multiple of 16
    (ctypes.c_void_p(0x1008), 1024, FAKE, EINVAL),  # misaligned
    (None, 0, None, OK),               # nothing to read
])
def test_read_bandwidth_validation(L, buf, nbytes, sink, code):
    """The measurement helper rejects bad arguments before any HIP call."""
    assert L.pkv_read_bandwidth(buf, nbytes, sink, None) == code


def test_python_layer_maps_statuses(L):
    import torch
    with pytest.raises((ValueError, TypeError)):
        pkv.paged_decode_partial(torch.zeros(2, 8, 128), None, None, None, None, 0.1, 2, 512, 128,
                                 None, None, None)


def _one_launch(L, **kw):
    a = dict(query=FAKE, dtype=1, kc=FAKE, vc=FAKE, layout=0, bt=FAKE, mb=8, lens=FAKE, S=2, H=8, KVH=2,
             D=128, bs=16, nb=64, scale=0.1, ps=64, ns=0, P=2, max_seq_len=128, acc=FAKE, m=FAKE, l=FAKE,
             ctr=FAKE, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return L.paged_decode(a["query"], a["dtype"], a["kc"], a["vc"], a["layout"], a["bt"], a["mb"], a["lens"],
                          a["S"], a["H"], a["KVH"], a["D"], a["bs"], a["nb"], a["scale"], a["ps"], a["ns"], a["P"],
                          a["max_seq_len"], a["acc"], a["m"], a["l"], a["ctr"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), EINVAL),                         # the one-launch decode needs out
    (dict(ctr=None), EINVAL),                         # more than one partition needs counters
    (dict(acc=None), EINVAL),                         # ... and the partial arrays
    (dict(ns=-1), EINVAL),
    (dict(ns=3, P=2), EINVAL),                        # fewer partitions than splits
    (dict(P=1, max_seq_len=128, ps=64, acc=None, m=None, l=None, out=None), EINVAL),
    (dict(bs=32, mb=16, ps=48), EINVAL),             # partition size not a multiple of block size 32
    (dict(D=96), EUNSUP),
    (dict(S=0), OK),                                  # empty batch: nothing to do
])
def test_one_launch_decode_validation(L, kw, code):
    assert _one_launch(L, **kw) == code, L.pkv_last_error()


def test_one_launch_single_pass_needs_no_partials(L):
    # one partition per sequence: NULL partials and counters pass validation; S = 0 keeps
    # the call from launching anything
    assert _one_launch(L, P=1, acc=None, m=None, l=None, ctr=None, S=0) == OK


def test_split_entry_points_validation(L):
    args = [FAKE, 1, FAKE, FAKE, 0, FAKE, 8, FAKE, 2, 8, 2, 128, 16, 64, 0.1]
    assert L.paged_decode_split_partial(*args, 0, 128, FAKE, FAKE, FAKE, None) == EINVAL   # num_splits = 0
    assert L.paged_decode_split_partial(*args, 4, 200, FAKE, FAKE, FAKE, None) == EINVAL   # max_seq_len > table
    args[12] = 0
    assert L.paged_decode_split_partial(*args, 4, 128, FAKE, FAKE, FAKE, None) == EINVAL   # block_size 0
    assert L.paged_decode_split_reduce(FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 0, FAKE, 1, None, None) == EINVAL
    assert L.paged_decode_split_reduce(FAKE, FAKE, FAKE, FAKE, 2, 8, 96, 16, 4, FAKE, 1, None, None) == EUNSUP
    assert L.paged_decode_split_reduce(FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 16, 4, FAKE, 1, None, None) == OK


def test_paged_attention_v2_validation(L):
    def call(alibi=None, D=128, bs=16, P=1, max_seq_len=512, H=8, dtype=1, kv_dtype=1, ks=1.0, vs=1.0):
        return L.paged_attention_v2(FAKE, FAKE, FAKE, FAKE, FAKE, dtype, FAKE, FAKE, 2, 0.1, FAKE, 32, FAKE, 2, H, D, bs,
                                    64, max_seq_len, P, alibi, kv_dtype, ks, vs, None)
    assert call(P=1, max_seq_len=513) == EINVAL  # 512-token partitions: 513 tokens need two
    assert call(H=7) == EINVAL               # 7 heads over 2 kv heads
    assert call(D=96) == EUNSUP
    assert call(kv_dtype=0) == EINVAL           # an f32 cache under a bf16 query
    assert call(ks=2.0) == EINVAL               # scales belong to a float8 cache
    assert call(kv_dtype=2, dtype=0) == EUNSUP  # a float8 cache needs a bf16 query
    assert call(kv_dtype=2, H=36) == EUNSUP     # ... and at most 16 query heads per kv head
    with pytest.raises(NotImplementedError):
        pkv.paged_attention_v2(None, None, None, None, None, None, None, 2, 0.1, None, None, 16, 0,
                               kv_cache_dtype="int4")


def test_mla_pages_validation(L):
    def call(ps=16, heads=16, tok_rows=FAKE, batch=2, total_q=4, num_pages=8, n_idx=4):
        return L.mla_paged_prefill_pages(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, batch, total_q, 2, num_pages,
                                         n_idx, heads, 512, 64, ps, 0.1, FAKE, tok_rows, FAKE, FAKE, None)
    assert call(ps=0) == EINVAL
    assert call(heads=8) == EUNSUP
    assert call(tok_rows=None) == EINVAL
    assert call(ps=1 << 20, num_pages=4096) == EUNSUP   # 2^32 pool rows
    assert call(batch=0) == OK


def test_mla_decode_validation(L):
    def call(heads=16, split=256, P=4, max_kv=1000, batch=2, num_pages=8, ps=1, acc=FAKE):
        return L.mla_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, batch, num_pages, 8, max_kv, heads, 512, 64, ps,
                                  0.1, split, P, acc, FAKE, FAKE, None, FAKE, FAKE, None)
    assert call(heads=8) == EUNSUP
    assert call(ps=16) == EUNSUP
    assert call(split=0) == EINVAL
    assert call(P=3) == EINVAL            # ceil(1000 / 256) = 4 splits
    assert call(acc=None) == EINVAL
    assert call(num_pages=0) == EINVAL
    assert call(batch=0) == OK


def test_cache_option_entry_points_validation(L):
    """paged_decode_partial_ex / paged_decode_ex: the cache options are checked before any
    launch (every call below fails validation or is an empty batch)."""
    def part(kv_dtype=1, ks=1.0, vs=1.0, dtype=1, S=2, H=8, kvh=2, ns=0, ps=512, P=1, mx=512):
        return L.paged_decode_partial_ex(FAKE, dtype, FAKE, FAKE, 0, kv_dtype, ks, vs, None, FAKE, 32, FAKE, S, H,
                                         kvh, 128, 16, 64, 0.1, ps, ns, P, mx, FAKE, FAKE, FAKE, None)

    def one(kv_dtype=1, ks=1.0, vs=1.0, dtype=1, out=FAKE, S=2):
        return L.paged_decode_ex(FAKE, dtype, FAKE, FAKE, 0, kv_dtype, ks, vs, None, FAKE, 32, FAKE, S, 8, 2, 128, 16,
                                 64, 0.1, 512, 0, 1, 512, None, None, None, None, out, None, None)
    assert part(kv_dtype=0) == EINVAL           # an f32 cache under a bf16 query
    assert part(kv_dtype=5) == EINVAL           # no such element type
    assert part(ks=0.5) == EINVAL               # scales belong to a float8 cache
    assert part(kv_dtype=2, ks=float("inf")) == EINVAL
    assert part(kv_dtype=2, dtype=0) == EUNSUP  # a float8 cache needs a bf16 query
    assert part(kv_dtype=2, H=36) == EUNSUP     # 18 query heads per kv head
    assert part(ps=24) == EINVAL                # not a multiple of the block size
    assert part(ns=4, P=2) == EINVAL            # fewer partial rows than splits
    assert part(P=1, mx=513) == EINVAL          # 513 tokens need two 512-token partitions
    assert part(kv_dtype=2, S=0) == OK          # empty batch
    assert one(out=None) == EINVAL
    assert one(kv_dtype=0) == EINVAL
    assert one(kv_dtype=2, dtype=0) == EUNSUP
    assert one(kv_dtype=2, S=0) == OK
