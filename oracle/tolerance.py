"""Elementwise error bound of the GPU path against the oracle.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the parity tests and
``__graft_entry__.smoke()`` use it to decide how far a GPU output may lie from
the oracle's on inputs outside the five workloads (which are held to the
flat 1e-2 / 1e-3).  It holds no step of the method; it prices the rounding
of the HIP path's arithmetic: bf16 inputs (exact), fp32 scores and sums, bf16
probabilities for the PV product, one bf16 rounding of the output.
"""
from __future__ import annotations

import numpy as np

from . import mla_oracle as oracle

# Unit roundoff of round-to-nearest-even: bf16 keeps 8 significant bits
# (7 stored + the implicit one), fp32 keeps 24.
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def row_out_bound(qrows, keys, scale):
    """Elementwise bound on |out_gpu - out_oracle| for query rows ``qrows``
    (float64 [R, 576]) over the keys they see (float64 [n, 576]), from the
    arithmetic of the HIP path (bf16 inputs, fp32 accumulation):

    * P is rounded to bf16 for the PV product while the row sum keeps fp32:
      each weight moves by <= U_BF16 relative, so column c moves by
      <= U_BF16 * A[c], A[c] = sum_t w_t |V_t[c]| (w = the softmax weights);
    * the fp32 scores carry <= 576 * U_F32 * softmax_scale * sum_d |q_d k_d|
      (any order of the 576-term sum) plus fp32 rounding of the scaled
      score, the exp2 and the base-2 references (<= 2^-16 in all, in natural-log
      units): Delta.  Weights then move by <= e^(2 Delta) - 1 ~ 2 Delta
      relative, i.e. <= 2 Delta * A[c] on column c;
    * the output is rounded to bf16 once: <= U_BF16 * |out|.

    Returns float64 [R, 512]: U_BF16 |ref| + (1 + U_BF16)(U_BF16 + 2.01 Delta) A + 1e-7."""
    R = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.full((R, 512), 1e-7)
    S = (qrows @ keys.T) * scale
    m = S.max(axis=1, keepdims=True)
    w = np.exp(S - m)
    w /= w.sum(axis=1, keepdims=True)
    vabs = np.abs(keys[:, :512])
    A = w @ vabs
    ref = np.abs(w @ keys[:, :512])
    mag = (np.abs(qrows) @ np.abs(keys).T).max(axis=1, keepdims=True)
    delta = scale * 576 * U_F32 * mag + np.abs(S).max(axis=1, keepdims=True) * 2 * U_F32 + 2.0 ** -16
    return U_BF16 * ref + (1 + U_BF16) * (U_BF16 + 2.01 * delta) * A + 1e-7


def dense_out_bound(inp, causal=False, kv=None):
    """row_out_bound for every (request, query token, head) of a dense decode,
    as float64 [b, s_q, h_q, 512]; ``kv`` replaces inp.kv_cache (the
    dequantized cache of an FP8 test)."""

    kv = inp.kv_cache if kv is None else kv
    b, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    tol = np.empty((b, s_q, h_q, 512))
    for i in range(b):
        L = int(inp.cache_seqlens[i])
        keys = oracle.request_keys(kv, inp.block_table[i], L)
        for s in range(s_q):
            n = L if not causal else max(0, L - (s_q - 1 - s))
            tol[i, s] = row_out_bound(oracle.bf16_to_f64(inp.q[i, s]), keys[:n], inp.softmax_scale)
    return tol


def sparse_out_bound(inp, indices=None, topk_length="inp", kv=None):
    """row_out_bound for every (request, query token, head) of a sparse decode."""

    idx = inp.indices if indices is None else indices
    tl = inp.topk_length if isinstance(topk_length, str) else topk_length
    kv = inp.kv_cache if kv is None else kv
    b, s_q, topk = idx.shape
    tol = np.empty((b, s_q, inp.q.shape[2], 512))
    for i in range(b):
        n = topk if tl is None else min(max(int(tl[i]), 0), topk)
        for s in range(s_q):
            keys = oracle.sparse_keys(kv, idx[i, s], n)
            tol[i, s] = row_out_bound(oracle.bf16_to_f64(inp.q[i, s]), keys, inp.softmax_scale)
    return tol
