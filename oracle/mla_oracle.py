"""CPU oracle for dense and sparse MLA decode (weight-absorbed, paged).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``.  The GPU library never links, imports or falls back to it, and it
shares no code with the GPU path: its only inputs are the seeded arrays that
``decode_attention_mla_amd.workloads`` draws.

Arithmetic is float64 throughout (bf16 inputs widen exactly).  The
functions follow these passages (page titles as on the web):

* "[DeepSeek-3] FlashMLA" (xutianle.me), section 3: the reference computation
  score = q @ kv[..., :576]^T, score *= softmax_scale, prob = softmax(score),
  out = prob @ kv[..., :512]; out is [b, s_q, h_q, 512], lse is [b, h_q, s_q].
* same page, section 4: a request's logical page j lives in physical block
  block_table[b][j]; cache_seqlens[b] is the number of valid tokens.
* "3.4 Attention kernel" (liuzhe1218.github.io), section on online softmax:
  running (m, l, o~) updated with the factor e^(m - m') when the max grows,
  and the merge of two partial states over disjoint key sets.
* same page, FlashAttention section: the log-sum-exp written out is m + log l.
* "[DeepSeek-3] FlashMLA", section 7, and the split-KV blog (0539edu.com),
  section 3.2/3.3: a split whose key set is empty (l = 0, m = -inf) is
  skipped in the merge; if every split is empty the output is 0.

Readings of points the pages leave open (each one is listed with its
justification in the design notes):
  * softmax_scale multiplies the scores (the overview's reference code);
  * lse is the natural log of sum(exp(scaled scores));
  * an empty request (L = 0) gives out = 0 and lse = -inf;
  * by default queries are not causally masked: every query token sees all
    L keys.  With ``causal=True`` (the API's is_causal flag, for multi-token
    prediction, s_q > 1) the s_q query tokens are the last s_q positions of
    the sequence, so query token s (0-based) sees keys 0 .. L - s_q + s, i.e.
    the first max(0, L - (s_q - 1 - s)) keys; a token that sees no key gets
    out = 0 and lse = -inf (the split-KV blog's note on splits whose keys are
    all masked).

Pins (tests/test_oracle.py): closed forms for L = 1, identical scores and
softmax_scale = 0, a position-encoded cache under uniform weights, the
worked QK partial sums printed on the multi-rail GEMM page, the e^(3-5)
rescale printed on the attention-kernel page, page-permutation invariance,
linearity, naive = online = split-then-merge, and brute force in exact
rational arithmetic on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 64
D_QK = 576
D_V = 512


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def request_keys(kv_cache: np.ndarray, block_table_row: np.ndarray, L: int) -> np.ndarray:
    """Gather the L valid cache rows of one request, in logical order.

    Logical token t sits in page block_table_row[t // 64] at slot t % 64
    (overview page, section 4).  Returns float64 [L, 576]; rows 0..L-1 only,
    so tail slots of the last page and unused table entries are never read.
    """
    L = int(L)
    if L == 0:
        return np.zeros((0, D_QK), dtype=np.float64)
    npages = (L + PAGE - 1) // PAGE
    pages = kv_cache[np.asarray(block_table_row[:npages], dtype=np.int64)]  # [n, 64, 1, 576]
    rows = pages.reshape(npages * PAGE, D_QK)[:L]
    return bf16_to_f64(rows)


def attend(qrows: np.ndarray, keys: np.ndarray, softmax_scale: float):
    """Softmax attention of R query rows over one request's keys.

    qrows float64 [R, 576]; keys float64 [L, 576] (V = keys[:, :512]).
    Returns (out [R, 512], lse [R]).  Plain definition: scores over all 576
    dims times softmax_scale, max-subtracted exponentials, normalised sum of
    the first 512 dims.
    """
    R = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((R, D_V)), np.full(R, -np.inf)
    scores = (qrows @ keys.T) * softmax_scale          # [R, L]
    m = scores.max(axis=1)
    p = np.exp(scores - m[:, None])
    l = p.sum(axis=1)
    out = (p @ keys[:, :D_V]) / l[:, None]
    lse = m + np.log(l)
    return out, lse


def visible_keys(L: int, s_q: int, s: int, causal: bool) -> int:
    """Number of keys query token s of s_q sees (see the causal reading above)."""
    return int(L) if not causal else max(0, int(L) - (s_q - 1 - s))


def mla_decode(q, kv_cache, block_table, cache_seqlens, softmax_scale, requests=None, causal=False):
    """Dense MLA decode for every (request, query token, head).

    q uint16 [b, s_q, h_q, 576] (bf16 bits); kv_cache uint16 [nb, 64, 1, 576];
    block_table int32 [b, max_blocks]; cache_seqlens int32 [b].
    Returns out float64 [b, s_q, h_q, 512] and lse float64 [b, h_q, s_q].
    ``requests`` restricts the work to a subset of request indices (the
    other entries are left as NaN).  ``causal`` masks each query token to the
    keys before and at its own position.
    """
    b, s_q, h_q, d = q.shape
    assert d == D_QK
    out = np.full((b, s_q, h_q, D_V), np.nan)
    lse = np.full((b, h_q, s_q), np.nan)
    todo = range(b) if requests is None else requests
    for i in todo:
        keys = request_keys(kv_cache, block_table[i], int(cache_seqlens[i]))
        for s in range(s_q):
            qrows = bf16_to_f64(q[i, s])                       # [h_q, 576]
            o, ls = attend(qrows, keys[:visible_keys(cache_seqlens[i], s_q, s, causal)], softmax_scale)
            out[i, s] = o
            lse[i, :, s] = ls
    return out, lse


def mla_decode_rows(q, kv_cache, block_table, cache_seqlens, softmax_scale, picks, causal=False):
    """Outputs for a sample of (request, query token, head) triples.

    Returns out float64 [n, 512] and lse float64 [n] in the order of ``picks``.
    """
    outs, lses = [], []
    cache = {}
    s_q = q.shape[1]
    for (i, s, h) in picks:
        if i not in cache:
            cache[i] = request_keys(kv_cache, block_table[i], int(cache_seqlens[i]))
        keys = cache[i][:visible_keys(cache_seqlens[i], s_q, s, causal)]
        o, ls = attend(bf16_to_f64(q[i, s, h])[None, :], keys, softmax_scale)
        outs.append(o[0])
        lses.append(ls[0])
    return np.array(outs), np.array(lses)


# ---------------------------------------------------------------------------
# Sparse (top-k) decode ("[DeepSeek-3] FlashMLA", section 11): each query
# token attends only to the cache rows its index list names; an entry is
# page_id * 64 + offset, the row at slot `offset` of physical block
# `page_id`, so no block table is involved.  Readings (listed in the design
# notes): the list is a multiset (an index named twice is two keys); only the
# first topk_length[b] entries of request b's lists count (the API's
# topk_length, which the overview names among the values that set the work;
# all topk entries when it is absent); an entry outside [0, num_blocks * 64),
# -1 padding for example, names no key; a query token left with no key gets
# out = 0 and lse = -inf, as an empty dense request does.

def sparse_keys(kv_cache: np.ndarray, index_row: np.ndarray, n_valid: int) -> np.ndarray:
    """The keys one query token's index list names, in list order.

    kv_cache uint16 [nb, 64, 1, 576]; index_row int [topk]; only entries
    0 .. n_valid - 1 count.  Returns float64 [k, 576].
    """
    rows = kv_cache.reshape(-1, D_QK)          # row page_id * 64 + offset
    picked = [int(e) for e in np.asarray(index_row)[:max(0, int(n_valid))] if 0 <= int(e) < rows.shape[0]]
    if not picked:
        return np.zeros((0, D_QK), dtype=np.float64)
    return bf16_to_f64(rows[np.asarray(picked, dtype=np.int64)])


def sparse_valid(topk: int, topk_length, i: int) -> int:
    """Entries of request i's index lists that count (see the reading above)."""
    if topk_length is None:
        return topk
    return min(max(int(topk_length[i]), 0), topk)


def mla_decode_sparse(q, kv_cache, indices, softmax_scale, topk_length=None):
    """Sparse MLA decode for every (request, query token, head).

    q uint16 [b, s_q, h_q, 576]; kv_cache uint16 [nb, 64, 1, 576];
    indices int32 [b, s_q, topk]; topk_length int32 [b] or None.
    Returns out float64 [b, s_q, h_q, 512] and lse float64 [b, h_q, s_q].
    """
    b, s_q, h_q, d = q.shape
    assert d == D_QK and indices.shape[:2] == (b, s_q)
    topk = indices.shape[2]
    out = np.full((b, s_q, h_q, D_V), np.nan)
    lse = np.full((b, h_q, s_q), np.nan)
    for i in range(b):
        n = sparse_valid(topk, topk_length, i)
        for s in range(s_q):
            o, ls = attend(bf16_to_f64(q[i, s]), sparse_keys(kv_cache, indices[i, s], n), softmax_scale)
            out[i, s] = o
            lse[i, :, s] = ls
    return out, lse


def mla_decode_sparse_rows(q, kv_cache, indices, softmax_scale, picks, topk_length=None):
    """Sparse outputs for a sample of (request, query token, head) triples:
    out float64 [n, 512] and lse float64 [n] in the order of ``picks``."""
    topk = indices.shape[2]
    outs, lses = [], []
    for (i, s, h) in picks:
        keys = sparse_keys(kv_cache, indices[i, s], sparse_valid(topk, topk_length, i))
        o, ls = attend(bf16_to_f64(q[i, s, h])[None, :], keys, softmax_scale)
        outs.append(o[0])
        lses.append(ls[0])
    return np.array(outs), np.array(lses)


# ---------------------------------------------------------------------------
# FP8 cache ("[DeepSeek-3] FlashMLA", section 12).  A token's record is 656
# bytes: the 512 latent dims as float8 e4m3, four fp32 scales (scale i covers
# dims 128 i .. 128 i + 127), the 64 RoPE dims as bf16.  The kernel
# dequantizes the latent to bf16 and joins the bf16 RoPE; QK^T and PV then
# run on bf16 inputs.  Reading (listed in the design notes): a latent value
# is bf16_rne(fp32(e4m3 * scale)) -- the product rounded to fp32, then to
# bf16 --, so the method on an FP8 cache is the bf16 method on that
# dequantized cache.  e4m3 is the OCP format (bias 7, no infinities, S.1111.111
# is NaN).

RECORD_FP8 = 656


def e4m3_value(byte: int) -> float:
    """One OCP e4m3 byte as a float (bias 7; subnormals below exponent 1)."""
    b = int(byte) & 0xFF
    sign = -1.0 if b & 0x80 else 1.0
    exp, man = (b >> 3) & 0xF, b & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * math.ldexp(man, -9)             # man/8 * 2^-6
    return sign * math.ldexp(8 + man, exp - 10)       # (1 + man/8) * 2^(exp-7)


def _f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def dequantize_fp8_cache(kv_fp8: np.ndarray) -> np.ndarray:
    """uint8 [nb, 64, 1, 656] records -> the bf16 cache (uint16 bit patterns
    [nb, 64, 1, 576]) the method computes with."""
    nb = kv_fp8.shape[0]
    rec = np.asarray(kv_fp8, np.uint8).reshape(nb * PAGE, RECORD_FP8)
    table = np.array([e4m3_value(b) for b in range(256)])
    lat = table[rec[:, :D_V]]                                           # float64, exact
    scale = rec[:, D_V:D_V + 16].copy().view(np.float32).astype(np.float64)   # [n, 4]
    prod = np.float32(1) * (lat.reshape(-1, 4, 128) * scale[:, :, None]).astype(np.float32)  # fp32 rounding
    out = np.empty((nb * PAGE, D_QK), np.uint16)
    out[:, :D_V] = _f32_to_bf16_rne(prod.reshape(-1, D_V))
    out[:, D_V:] = rec[:, D_V + 16:].copy().view(np.uint16)
    return out.reshape(nb, PAGE, 1, D_QK)


# ---------------------------------------------------------------------------
# Online softmax and the merge of partial states (attention-kernel page,
# online-softmax section; overview page, section 7).

def online_attend(qrows: np.ndarray, keys: np.ndarray, softmax_scale: float, block: int = PAGE):
    """Same result as ``attend`` reached block by block with running (m, l, o~).

    For each key block: m' = max(m, blockmax), l' = e^(m-m') l + sum e^(s-m'),
    o~' = e^(m-m') o~ + sum e^(s-m') v; at the end out = o~ / l and
    lse = m + log l.
    """
    R = qrows.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, D_V))
    for j in range(0, keys.shape[0], block):
        kb = keys[j:j + block]
        s = (qrows @ kb.T) * softmax_scale
        m_new = np.maximum(m, s.max(axis=1))
        scale_old = np.exp(m - m_new)          # e^(m - m'), 0 on the first block
        p = np.exp(s - m_new[:, None])
        l = scale_old * l + p.sum(axis=1)
        acc = scale_old[:, None] * acc + p @ kb[:, :D_V]
        m = m_new
    if keys.shape[0] == 0:
        return np.zeros((R, D_V)), np.full(R, -np.inf)
    return acc / l[:, None], m + np.log(l)


def rescale_factor(m_old: float, m_new: float) -> float:
    """Factor applied to the old running sum and output when the max moves."""
    return math.exp(m_old - m_new)


def merge_partials(outs: np.ndarray, lses: np.ndarray):
    """Merge split results (normalised O_i, lse_i) over disjoint key sets.

    outs [n, R, 512], lses [n, R].  With M = max_i lse_i and w_i = e^(lse_i - M):
    out = sum_i w_i O_i / sum_i w_i, lse = M + log sum_i w_i.  Splits with
    lse_i = -inf (empty key set) get weight 0; if all are empty, out = 0 and
    lse = -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)                                # [R]
    empty = np.isneginf(M)
    Ms = np.where(empty, 0.0, M)
    w = np.exp(lses - Ms[None, :])                       # exp(-inf) = 0
    wsum = w.sum(axis=0)
    safe = np.where(empty, 1.0, wsum)
    out = np.einsum("nr,nrc->rc", w, outs) / safe[:, None]
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, Ms + np.log(safe))
    return out, lse


def split_then_merge(qrows: np.ndarray, keys: np.ndarray, softmax_scale: float, bounds):
    """Attend separately over keys[bounds[k]:bounds[k+1]] and merge the parts."""
    outs, lses = [], []
    for a, e in zip(bounds[:-1], bounds[1:]):
        o, ls = attend(qrows, keys[a:e], softmax_scale)
        outs.append(o)
        lses.append(ls)
    return merge_partials(np.stack(outs), np.stack(lses))
