"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

try:
    from hypothesis import given, settings, strategies as st
    HAVE_HYPOTHESIS = True
except ImportError:  # pragma: no cover
    HAVE_HYPOTHESIS = False


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


if HAVE_HYPOTHESIS:
    @settings(max_examples=40, deadline=None)
    @given(st.data())
    def test_decode_sweep_against_brute_force(data):
        S = data.draw(st.integers(1, 3))
        KVH = data.draw(st.integers(1, 3))
        G = data.draw(st.integers(1, 3))
        D = data.draw(st.sampled_from([4, 8, 16]))
        bs = data.draw(st.sampled_from([1, 2, 4, 16]))
        lens = [data.draw(st.integers(0, 70)) for _ in range(S)]
        layout = data.draw(st.sampled_from(["token_major", "xpacked"]))
        ps = bs * data.draw(st.integers(1, 5))
        seed = data.draw(st.integers(0, 2**31 - 1))
        q, kc, vc, bt, lens_a, K, V = pins._tiny_case(seed, lens, KVH * G, KVH, D, bs, layout)
        out, lse = oracle.decode(q, kc, vc, layout, bt, lens_a, 0.25, KVH, bs)
        ref_out, ref_lse = pins._brute_decode(q, K, V, lens_a, 0.25, G)
        pins._close(out, ref_out, 1e-12, what="sweep out")
        pins._close(lse, ref_lse, 1e-12, what="sweep lse")
        P = max(1, -(-max(lens) // ps))
        acc, m, l = oracle.decode_partials(q, kc, vc, layout, bt, lens_a, 0.25, KVH, bs, ps, P)
        o2, s2 = oracle.reduce_partials(acc, m, l, lens_a, ps)
        pins._close(o2, ref_out, 1e-12, what="sweep split out")
        pins._close(s2, ref_lse, 1e-12, what="sweep split lse")

    @settings(max_examples=25, deadline=None)
    @given(st.data())
    def test_mla_sweep_against_sdpa(data):
        B = data.draw(st.integers(1, 3))
        q_lens = [data.draw(st.integers(1, 6)) for _ in range(B)]
        prefixes = [data.draw(st.integers(0, 9)) for _ in range(B)]
        seed = data.draw(st.integers(0, 2**31 - 1))
        qn, qp, ckv, kpe, qo, kv, idx = pins._mla_tiny(seed, q_lens, prefixes, H=2, Dc=4, Dp=2)
        O, L = oracle.mla_prefill(qn, qp, ckv, kpe, qo, kv, idx, 0.6)
        for b in range(B):
            r0, r1 = qo[b], qo[b + 1]
            ro, rl = pins._sdpa_rows(qn[r0:r1], qp[r0:r1], ckv, kpe, idx[kv[b]:kv[b + 1]], r1 - r0, 0.6)
            pins._close(O[r0:r1], ro, 1e-12, what="mla sweep O")
            pins._close(L[r0:r1], rl, 1e-12, what="mla sweep lse")
