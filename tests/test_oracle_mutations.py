"""Planted mistakes in the oracle must each be caught by at least one pin.

Every mutant is a copy of the ``oracle`` package with one textual change (a dropped
term, a wrong sign or index, a swapped operand, the other page's reading). The pins in
``oracle_pins.py`` run against the mutant; the test passes only if one of them fails.
Nothing here touches the GPU or the HIP library.
"""
import ast
import importlib
import os
import shutil
import sys

import pytest

from tests import oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# (file, original snippet, replacement, occurrence index, description)
MUTATIONS = [
    ("decode.py", "return h // group", "return h % group", 0, "kv head index h % G"),
    ("decode.py", "off = t % block_size", "off = (t + 1) % block_size", 0, "slot off by one"),
    ("decode.py", "K[h] = _index(key_cache, (blk, h, off, slice(None)))",
     "K[h] = _index(key_cache, (blk, 0, off, slice(None)))", 0, "token-major K always head 0"),
    ("decode.py", "V[h] = _index(value_cache, (blk[:, None], h, d[None, :], off[:, None]))",
     "V[h] = _index(value_cache, (blk[:, None], h, (d_model - 1 - d)[None, :], off[:, None]))", 0,
     "x-packed V dim reversed"),
    ("decode.py", "(d // x)[None, :], off[:, None], (d % x)[None, :]",
     "(d % x * 0 + d // x)[None, :], off[:, None], (x - 1 - d % x)[None, :]", 0, "x-packed K lane reversed"),
    ("decode.py", "s = scale * (K @ q_vec)", "s = (K @ q_vec)", 0, "scale dropped"),
    ("decode.py", "out[b, h] = (e @ V[kh]) / Z", "out[b, h] = (e @ V[kh])", 0, "normalization dropped"),
    ("decode.py", "lse[b, h] = M + np.log(Z)", "lse[b, h] = np.log(Z)", 0, "max term dropped from lse"),
    ("decode.py", "acc[b, h, p] = e @ V[kh][t0:t1]", "acc[b, h, p] = (e @ V[kh][t0:t1]) / e.sum()", 0,
     "normalized partial acc"),
    ("decode.py", "return [(p * span, min((p + 1) * span, n)) for p in range(count)]",
     "return [(p * span, min((p + 1) * span, n - 1)) for p in range(count)]", 0,
     "last token dropped from partition"),
    ("decode.py", "m[b, h, p] = mp", "m[b, h, p] = mp * np.log2(np.e)", 0, "partial m in base 2"),
    ("decode.py", "w = np.exp(mp - M)", "w = np.exp(M - mp)", 0, "combine weight sign"),
    ("decode.py", "Z = w @ l[b, h, :nparts]", "Z = w.sum()", 0, "exp-sums dropped from combine"),
    ("decode.py", "lse[b, h] = M + np.log(Z)", "lse[b, h] = np.log(Z)", 1, "max term dropped from reduce lse"),
    ("decode.py", "count = -(-n // span)", "count = max(1, n // span)", 0, "floor partition count"),
    ("decode.py", "bps = -(-nb // num_splits)", "bps = max(1, nb // num_splits)", 0, "floor pages per split"),
    ("decode.py", "span = bps * block_size", "span = bps * block_size - 1", 0, "split span one token short"),
    ("decode.py", "nb = -(-n // block_size)", "nb = max(1, n // block_size)", 0, "floor page count of a split"),
    ("decode.py", "acc[b, h, p] = acc[b, h, p] / l[b, h, p]", "acc[b, h, p] = acc[b, h, p] * 1.0", 0,
     "normalized partial not divided by l"),
    ("decode.py", "out[b, h] = ((w * l[b, h, :nparts]) @ acc[b, h, :nparts]) / Z",
     "out[b, h] = (w @ acc[b, h, :nparts]) / Z", 0, "normalized reduce without exp-sums weight"),
    ("decode.py", "s = s - float(slope) * ((n - 1) - np.arange(n))", "s = s + float(slope) * ((n - 1) - np.arange(n))",
     0, "ALiBi sign"),
    ("decode.py", "s = s - float(slope) * ((n - 1) - np.arange(n))", "s = s - float(slope) * (n - np.arange(n))", 0,
     "ALiBi query position n instead of n - 1"),
    ("decode.py", "s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[h])",
     "s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[kh])", 0, "ALiBi slope of the kv head"),
    ("decode.py", "K, V = _dequant(K, k_scale), _dequant(V, v_scale)\n        for h in range(H):\n            kh = _kv_head(h, G)\n            s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[h])\n            M = s.max()",
     "K, V = _dequant(K, v_scale), _dequant(V, k_scale)\n        for h in range(H):\n            kh = _kv_head(h, G)\n            s = _scores(q[b, h], K[kh], scale, None if slopes is None else slopes[h])\n            M = s.max()",
     0, "cache scales swapped"),
    ("decode.py", "return x * float(cache_scale)", "return x", 0, "cache scale dropped"),
    ("mla.py", "vis = min(prefix + i + 1, kv_len)", "vis = min(prefix + i, kv_len)", 0, "causal off by one"),
    ("mla.py", "return sm_scale * (qn_row @ Kc.T + qp_row @ Kp.T)", "return sm_scale * (qn_row @ Kc.T)", 0,
     "kpe term dropped"),
    ("mla.py", "lse2[r] = (M[:, 0] + np.log(Z[:, 0])) / ln2", "lse2[r] = (M[:, 0] + np.log(Z[:, 0]))", 0,
     "natural-log lse"),
    ("mla.py", "prefix = kv_len - q_len\n", "prefix = 0\n", 0, "top-left causal alignment"),
    ("mla.py", "Kc = ckv[pages[j // ps], j % ps, :]", "Kc = ckv[np.sort(pages)[j // ps], j % ps, :]", 0,
     "kv_indices order ignored"),
    ("mla.py", "pages = idx[k0:k1]", "pages = idx[q0:q0 + n_pages]", 0, "qo_indptr used for keys"),
    ("mla.py", "Kc = ckv[pages[j // ps], j % ps, :]", "Kc = ckv[pages[j // ps], (j + 1) % ps, :]", 0,
     "page slot off by one"),
    ("mla.py", "Kp = kpe[pages[j // ps], j % ps, :]", "Kp = kpe[pages[j // ps], 0, :]", 0, "kpe from slot 0"),
    ("mla.py", "(n_pages - 1) * ps + last", "n_pages * ps", 0, "last page length ignored"),
    ("mla.py", "Kc = ckv[pages[j // ps], j % ps, :]", "Kc = ckv[pages[j % ps], j % ps, :]", 0,
     "page index from the slot"),
    ("mla.py", "O[r] = (e @ Kc[:vis]) / Z", "O[r] = (e @ Kc[:vis]) / Z.sum()", 0, "normalization across heads"),
]


def _code_only(src):
    """AST dump with docstrings removed, so a mutation that only edits prose is rejected."""
    tree = ast.parse(src)
    for node in ast.walk(tree):
        body = getattr(node, "body", None)
        if isinstance(body, list) and body and isinstance(body[0], ast.Expr) \
                and isinstance(getattr(body[0], "value", None), ast.Constant) \
                and isinstance(body[0].value.value, str):
            node.body = body[1:] or [ast.Pass()]
    return ast.dump(tree)


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"snippet not found: {old!r}"
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("idx", range(len(MUTATIONS)), ids=[m[4] for m in MUTATIONS])
def test_mutant_is_caught(idx, tmp_path):
    fname, old, new, nth, what = MUTATIONS[idx]
    pkg = f"oracle_mutant_{idx}"
    dst = tmp_path / pkg
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    path = dst / fname
    original = path.read_text()
    mutated = _replace_nth(original, old, new, nth)
    assert _code_only(mutated) != _code_only(original), f"mutation only touches prose: {what}"
    path.write_text(mutated)
    sys.path.insert(0, str(tmp_path))
    try:
        mutant = importlib.import_module(pkg)
        caught = []
        for pin in pins.ALL_PINS:
            try:
                pin(mutant)
            except Exception as e:  # AssertionError or a crash: either way the pin failed
                caught.append((pin.__name__, type(e).__name__))
        assert caught, f"no pin catches the planted mistake: {what}"
    finally:
        sys.path.remove(str(tmp_path))
        for k in [k for k in sys.modules if k == pkg or k.startswith(pkg + ".")]:
            del sys.modules[k]
