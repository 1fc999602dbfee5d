"""Streams and graph capture, through the binding (the C ABI takes a hipStream_t and
launches only there): a side stream gives the default stream's results bit for bit, two
batches launched interleaved on two streams each give their own results, and the two-phase
decode captured in a HIP graph gives the eager result on every replay, with new inputs and
other eager work between replays. All streams keep the default priority.
"""
import numpy as np
import pytest
import torch

import paged_kv_gqa_table_amd as pkv
from paged_kv_gqa_table_amd import inputs
from tests.test_parity_gpu import say

pytestmark = pytest.mark.gpu


def _decode_two_phase(case, q, kc, vc, bt, lens, outs):
    acc, m, l, out, lse = outs
    pkv.paged_decode_partial(q, kc, vc, bt, lens, case.scale, case.num_kv_heads, 512, case.max_seq_len, acc, m, l,
                             layout=case.layout)
    pkv.paged_decode_reduce(acc, m, l, lens, 512, out, lse)


def _bufs(case, dev="cuda"):
    S, H, D = case.num_seqs, case.num_heads, case.head_dim
    P = -(-case.max_seq_len // 512)
    return (torch.zeros((S, H, P, D), dtype=torch.float32, device=dev),
            torch.zeros((S, H, P), dtype=torch.float32, device=dev),
            torch.zeros((S, H, P), dtype=torch.float32, device=dev),
            torch.zeros((S, H, D), dtype=case.query.dtype, device=dev),
            torch.zeros((S, H), dtype=torch.float32, device=dev))


def _dev(case):
    return (case.query.cuda(), case.key_cache.cuda(), case.value_cache.cuda(), case.block_tables.cuda(),
            case.seq_lens.cuda())


def test_side_stream_same_bits():
    case = inputs.make_decode([1, 700, 1500, 2049, 0], 32, 8, 128, seed=61)
    t = _dev(case)
    say("side stream: GQA two-phase, one launch, MLA prefill and decode")
    ref = _bufs(case)
    _decode_two_phase(case, *t, ref)
    ref1 = pkv.paged_decode(*t[:4], t[4], case.scale, case.num_kv_heads, 512, layout=case.layout,
                            max_seq_len=case.max_seq_len, return_lse=True, one_launch=True)
    mla = inputs.make_mla(np.array([3, 40]), np.array([500, 70]), seed=62)
    mt = [getattr(mla, k).cuda() for k in ("q_nope", "q_pe", "ckv_cache", "kpe_cache", "qo_indptr", "kv_indptr",
                                          "kv_indices")]
    mref = pkv.mla_paged_prefill(*mt, mla.sm_scale)
    last = (mt[4][1:] - 1).long()
    dref = pkv.mla_paged_decode(mt[0][last].contiguous(), mt[1][last].contiguous(), mt[2], mt[3], mt[5], mt[6],
                                mla.sm_scale, split_tokens=128)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = _bufs(case)
        _decode_two_phase(case, *t, got)
        got1 = pkv.paged_decode(*t[:4], t[4], case.scale, case.num_kv_heads, 512, layout=case.layout,
                                max_seq_len=case.max_seq_len, return_lse=True, one_launch=True)
        mgot = pkv.mla_paged_prefill(*mt, mla.sm_scale)
        dgot = pkv.mla_paged_decode(mt[0][last].contiguous(), mt[1][last].contiguous(), mt[2], mt[3], mt[5], mt[6],
                                    mla.sm_scale, split_tokens=128)
    s.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b), "two-phase decode differs on a side stream"
    for a, b in zip(ref1, got1):
        assert torch.equal(a, b), "one-launch decode differs on a side stream"
    for a, b in zip(mref + dref, mgot + dgot):
        assert torch.equal(a, b), "MLA differs on a side stream"


def test_two_streams_interleaved():
    c1 = inputs.make_decode([300, 4096, 17, 900], 32, 8, 128, seed=63)
    c2 = inputs.make_decode([2000, 5, 1024], 24, 4, 256, layout="xpacked", seed=64)
    t1, t2 = _dev(c1), _dev(c2)
    say("two streams: two batches interleaved")
    r1, r2 = _bufs(c1), _bufs(c2)
    _decode_two_phase(c1, *t1, r1)
    _decode_two_phase(c2, *t2, r2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    g1, g2 = _bufs(c1), _bufs(c2)
    for rep in range(3):
        with torch.cuda.stream(s1):
            _decode_two_phase(c1, *t1, g1)
        with torch.cuda.stream(s2):
            _decode_two_phase(c2, *t2, g2)
    s1.synchronize()
    s2.synchronize()
    for a, b in zip(r1 + r2, g1 + g2):
        assert torch.equal(a, b), "interleaved streams changed a result"


def test_graph_replay_matches_eager():
    case = inputs.make_decode([1, 512, 513, 3000, 77, 0], 32, 8, 128, seed=65)
    q, kc, vc, bt, lens = _dev(case)
    rng = np.random.default_rng(66)
    outs = _bufs(case)
    say("graph capture of the two-phase decode, three replays")
    _decode_two_phase(case, q, kc, vc, bt, lens, outs)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_two_phase(case, q, kc, vc, bt, lens, outs)
    other = inputs.make_decode([1000, 200], 16, 2, 64, seed=67)
    ot = _dev(other)
    for rep in range(3):
        q.copy_(torch.from_numpy(rng.standard_normal(tuple(q.shape), dtype=np.float32)).to(q.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in outs]
        ob = _bufs(other)  # eager work between replays
        _decode_two_phase(other, *ot, ob)
        ref = _bufs(case)
        _decode_two_phase(case, q, kc, vc, bt, lens, ref)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"graph replay {rep} differs from the eager result"
