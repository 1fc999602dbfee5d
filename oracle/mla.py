"""Oracle for MLA causal paged prefill with a base-2 LSE (page_size 1, and pages of
several tokens).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the kernelindex page for the gemini-2.5-pro Triton MLA paged-prefill
kernel (``_mla_paged_prefill_causal_h16_ckv512_kpe64_ps1_kernel`` and its
``_forward`` host wrapper). What it computes, restated:
  * rows of batch b are qo_indptr[b] .. qo_indptr[b+1]-1, its keys are the tokens
    kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] (one token per page);
  * query i of the batch sits at absolute position prefix + i with
    prefix = kv_len - q_len, and sees keys j <= prefix + i (bottom-right causal);
  * logit x_j = sm_scale * (q_nope . ckv_j + q_pe . kpe_j);
  * O = softmax(x) applied to ckv only (kpe enters only the logits);
  * lse = log2 sum_j exp(x_j), i.e. the natural-log LSE divided by ln 2 (the
    page's closing comment of its first pass states this form; its prose about a
    log(2) factor is garbled and its code multiplies by log2(e));
  * kv_len = 0 gives O = 0 and lse = -inf (the page's empty-KV branch). More
    generally any row that sees no key (prefix + i < 0, which only a caller that
    breaks kv_len >= q_len can produce) gets O = 0 and lse = -inf.

Pages of ps > 1 tokens (the page's kernel takes a PAGE_SIZE but its host wrapper
asserts 1; the plainest reading of its page-counting kv_indptr): batch b owns pages
kv_indices[kv_indptr[b] .. kv_indptr[b+1]-1] in order, every page holds ps tokens
except the last, which holds kv_last_page_len[b] (ps when no such array is given);
key token j sits at slot j % ps of page kv_indices[kv_indptr[b] + j // ps].
"""
from __future__ import annotations

import math

import numpy as np

from .decode import _as_f64, _as_int


def _logits(qn_row: np.ndarray, qp_row: np.ndarray, Kc: np.ndarray, Kp: np.ndarray,
            sm_scale: float) -> np.ndarray:
    """x[h, j] = sm_scale * (q_nope[h] . ckv_j + q_pe[h] . kpe_j)."""
    return sm_scale * (qn_row @ Kc.T + qp_row @ Kp.T)


def mla_prefill(q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_indptr, kv_indices,
                sm_scale: float, kv_last_page_len=None):
    """Returns (O [total_q, H, ckv_dim], lse2 [total_q, H]) in float64.

    ckv_cache is [num_pages, ps, ckv_dim] and kpe_cache [num_pages, ps, kpe_dim]."""
    qn = _as_f64(q_nope)
    qp = _as_f64(q_pe)
    ckv = _as_f64(ckv_cache)
    kpe = _as_f64(kpe_cache)
    qo = _as_int(qo_indptr)
    kvp = _as_int(kv_indptr)
    idx = _as_int(kv_indices)
    ps = ckv.shape[1]
    if kpe.shape[1] != ps:
        raise ValueError("ckv and kpe pages must hold the same number of tokens")
    last_len = None if kv_last_page_len is None else _as_int(kv_last_page_len)
    total_q, H, Dc = qn.shape
    O = np.zeros((total_q, H, Dc))
    lse2 = np.full((total_q, H), -np.inf)
    ln2 = math.log(2.0)
    for b in range(len(qo) - 1):
        q0, q1 = int(qo[b]), int(qo[b + 1])
        k0, k1 = int(kvp[b]), int(kvp[b + 1])
        n_pages = k1 - k0
        last = ps if last_len is None else int(last_len[b])
        q_len, kv_len = q1 - q0, (n_pages - 1) * ps + last if n_pages > 0 else 0
        if q_len == 0 or kv_len == 0:
            continue
        pages = idx[k0:k1]
        j = np.arange(kv_len)
        Kc = ckv[pages[j // ps], j % ps, :]
        Kp = kpe[pages[j // ps], j % ps, :]
        prefix = kv_len - q_len
        for i in range(q_len):
            r = q0 + i
            vis = min(prefix + i + 1, kv_len)
            if vis <= 0:
                continue
            x = _logits(qn[r], qp[r], Kc[:vis], Kp[:vis], sm_scale)   # [H, vis]
            M = x.max(axis=1, keepdims=True)
            e = np.exp(x - M)
            Z = e.sum(axis=1, keepdims=True)
            O[r] = (e @ Kc[:vis]) / Z
            lse2[r] = (M[:, 0] + np.log(Z[:, 0])) / ln2
    return O, lse2
