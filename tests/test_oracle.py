"""Pins for the CPU oracle: closed forms, printed worked examples, invariants
and exact brute force.  None of these re-types the oracle's own formula; each
is chosen so that a plausible mistake (a dropped RoPE term, V taken from the
wrong dims, a wrong page or tail read, a flipped rescale sign, a broken merge)
fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from decode_attention_mla_amd import workloads as W
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D_QK, D_V, PAGE = 576, 512, 64


def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _single_request(keys_f32, q_f32, scale, pool_extra=3, seed=0):
    """Place one request's keys on randomly chosen physical pages."""
    L = keys_f32.shape[0]
    n = (L + PAGE - 1) // PAGE
    rng = np.random.default_rng(seed)
    pool = n + pool_extra
    perm = rng.permutation(pool)
    kv = np.full((pool, PAGE, 1, D_QK), W.POISON_BITS, dtype=np.uint16)
    for t in range(L):
        kv[perm[t // PAGE], t % PAGE, 0] = _bits(keys_f32[t])
    bt = np.full((1, max(n, 1) + 1), perm[-1], dtype=np.int32)
    bt[0, :n] = perm[:n]
    q = _bits(q_f32).reshape(1, 1, -1, D_QK)
    return q, kv, bt, np.array([L], dtype=np.int32)


def test_bf16_rounding_known_values():
    vals = np.array([1.0, -2.0, 1e4, 1.00390625, 1.01171875, 3.0e38], dtype=np.float32)
    bits = W.f32_to_bf16_bits(vals)
    # 1.00390625 = 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7: even mantissa wins (1.0).
    # 1.01171875 = 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even wins (1+2^-6).
    assert list(bits[:5]) == [0x3F80, 0xC000, 0x461C, 0x3F80, 0x3F82]
    back = W.bf16_bits_to_f32(bits)
    assert back[2] == 9984.0
    assert np.all(oracle.bf16_to_f64(bits) == back.astype(np.float64))


def test_worked_qk_partial_sums_from_multirail_page():
    g = json.load(open(os.path.join(GOLDEN, "multirail_qk_partial_sums.json")))
    # A single-token cache has lse = scale * q.k, so lse exposes the dot product.
    for where in (0, D_QK - 4):          # latent dims and the RoPE tail both count
        for key, half, expect in (("k1", None, g["full"]["k1"]), ("k2", None, g["full"]["k2"]),
                                  ("k1", 0, g["first_half"]["k1"]), ("k2", 0, g["first_half"]["k2"]),
                                  ("k1", 1, g["second_half"]["k1"]), ("k2", 1, g["second_half"]["k2"])):
            qv = np.zeros(D_QK, np.float32)
            qv[where:where + 4] = g["q"]
            if half == 0:
                qv[where + 2:where + 4] = 0
            elif half == 1:
                qv[where:where + 2] = 0
            k = np.zeros((1, D_QK), np.float32)
            k[0, where:where + 4] = g[key]
            q, kv, bt, sl = _single_request(k, qv[None, :], 1.0)
            out, lse = oracle.mla_decode(q, kv, bt, sl, 1.0)
            assert lse[0, 0, 0] == expect


def test_two_token_worked_example_softmax():
    g = json.load(open(os.path.join(GOLDEN, "multirail_qk_partial_sums.json")))
    qv = np.zeros(D_QK, np.float32)
    qv[:4] = g["q"]
    k = np.zeros((2, D_QK), np.float32)
    k[0, :4] = g["k1"]
    k[1, :4] = g["k2"]
    q, kv, bt, sl = _single_request(k, qv[None, :], 1.0)
    out, lse = oracle.mla_decode(q, kv, bt, sl, 1.0)
    # scores 70 and 10: lse = 70 + log(1 + e^-60); weights 1/(1+e^-60), e^-60/(1+e^-60)
    assert abs(lse[0, 0, 0] - (70.0 + math.log1p(math.exp(-60.0)))) < 1e-12
    w2 = math.exp(-60.0) / (1 + math.exp(-60.0))
    expect = (1 - w2) * np.array(g["k1"], float) + w2 * np.array(g["k2"], float)
    assert np.allclose(out[0, 0, 0, :4], expect, rtol=0, atol=1e-15)
    assert np.all(out[0, 0, 0, 4:] == 0)


def test_rescale_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_rescale.json")))
    assert abs(oracle.rescale_factor(g["m_old"], g["m_new"]) - math.exp(g["factor_log"])) < 1e-15
    # Two key blocks whose maxima are 3 then 5: the online result must equal the
    # closed form log(e^3 + e^1 + e^5 + e^2) only if the old state is scaled by e^(3-5).
    q = np.zeros((1, D_QK))
    q[0, 0] = 1.0
    keys = np.zeros((4, D_QK))
    keys[:, 0] = [3.0, 1.0, 5.0, 2.0]
    keys[:, 1] = [1.0, 2.0, 4.0, 8.0]        # V column 1 distinguishes the tokens
    out, lse = oracle.online_attend(q, keys, 1.0, block=2)
    z = math.exp(3) + math.exp(1) + math.exp(5) + math.exp(2)
    assert abs(lse[0] - math.log(z)) < 1e-12
    expect = (math.exp(3) * 1 + math.exp(1) * 2 + math.exp(5) * 4 + math.exp(2) * 8) / z
    assert abs(out[0, 1] - expect) < 1e-12


def test_single_token_cache_gives_v():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, D_QK)).astype(np.float32)
    qv = rng.standard_normal((16, D_QK)).astype(np.float32)
    scale = W.SOFTMAX_SCALE
    q, kv, bt, sl = _single_request(k, qv, scale)
    out, lse = oracle.mla_decode(q, kv, bt, sl, scale)
    v = W.bf16_bits_to_f32(_bits(k[0]))[:D_V].astype(np.float64)
    assert np.all(out[0, 0] == v[None, :])             # exactly v, every head
    kq = [Fraction(float(x)) for x in W.bf16_bits_to_f32(_bits(k[0]))]
    for h in range(16):
        qq = [Fraction(float(x)) for x in W.bf16_bits_to_f32(_bits(qv[h]))]
        dot = float(sum(a * b for a, b in zip(qq, kq)))
        assert abs(lse[0, h, 0] - scale * dot) < 1e-9


def _identical_scores_case(L, seed):
    """q latent part 0, every token shares one RoPE key, latent parts differ."""
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((L, D_QK)).astype(np.float32)
    keys[:, D_V:] = rng.standard_normal(D_QK - D_V).astype(np.float32)[None, :]
    qv = rng.standard_normal((4, D_QK)).astype(np.float32)
    qv[:, :D_V] = 0
    return keys, qv


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_identical_scores_give_mean_of_v(L):
    keys, qv = _identical_scores_case(L, seed=L)
    scale = W.SOFTMAX_SCALE
    q, kv, bt, sl = _single_request(keys, qv, scale, seed=L)
    out, lse = oracle.mla_decode(q, kv, bt, sl, scale)
    kb = W.bf16_bits_to_f32(_bits(keys)).astype(np.float64)
    qb = W.bf16_bits_to_f32(_bits(qv)).astype(np.float64)
    mean_v = np.array([math.fsum(kb[:, c]) / L for c in range(D_V)])
    assert np.allclose(out[0, 0], mean_v[None, :], rtol=0, atol=1e-12)
    for h in range(4):
        qr = math.fsum(float(a) * float(b) for a, b in zip(qb[h, D_V:], kb[0, D_V:]))
        assert abs(lse[0, h, 0] - (scale * qr + math.log(L))) < 1e-10


def test_literal_identical_keys_give_that_row():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(D_QK).astype(np.float32)
    keys = np.repeat(row[None, :], 77, axis=0)
    qv = rng.standard_normal((3, D_QK)).astype(np.float32)
    q, kv, bt, sl = _single_request(keys, qv, 0.3)
    out, lse = oracle.mla_decode(q, kv, bt, sl, 0.3)
    v = W.bf16_bits_to_f32(_bits(row))[:D_V].astype(np.float64)
    assert np.allclose(out[0, 0], v[None, :], rtol=0, atol=1e-13)


def test_zero_scale_gives_uniform_weights():
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((130, D_QK)).astype(np.float32)
    qv = rng.standard_normal((2, D_QK)).astype(np.float32)
    q, kv, bt, sl = _single_request(keys, qv, 0.0)
    out, lse = oracle.mla_decode(q, kv, bt, sl, 0.0)
    kb = W.bf16_bits_to_f32(_bits(keys)).astype(np.float64)
    assert np.allclose(out[0, 0], kb[:, :D_V].mean(axis=0)[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse[0, :, 0], math.log(130), rtol=0, atol=1e-13)


@pytest.mark.parametrize("L", [1, 64, 65, 128, 257])
def test_position_encoded_cache(L):
    """V encodes each token's logical position; uniform weights give the mean
    position, which only comes out right if the page table, slot order and
    tail length are all honoured."""
    keys = np.zeros((L, D_QK), np.float32)
    t = np.arange(L)
    keys[:, 0] = t                 # exact in bf16 for t <= 256
    keys[:, 1] = t % PAGE
    keys[:, 2] = t // PAGE
    qv = np.ones((1, D_QK), np.float32)
    q, kv, bt, sl = _single_request(keys, qv, 0.0, seed=L)
    out, _ = oracle.mla_decode(q, kv, bt, sl, 0.0)
    assert abs(out[0, 0, 0, 0] - (L - 1) / 2) < 1e-12
    assert abs(out[0, 0, 0, 1] - np.mean(t % PAGE)) < 1e-12
    assert abs(out[0, 0, 0, 2] - np.mean(t // PAGE)) < 1e-12


def test_page_shuffle_is_bitwise_invariant():
    inp = W.config_inputs(1)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale)
    rng = np.random.default_rng(11)
    perm = rng.permutation(inp.num_blocks)          # new physical home of each page
    kv2 = np.empty_like(inp.kv_cache)
    kv2[perm] = inp.kv_cache
    bt2 = perm[inp.block_table].astype(np.int32)
    out2, lse2 = oracle.mla_decode(inp.q, kv2, bt2, inp.cache_seqlens, inp.softmax_scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_linear_in_latent_values_for_rope_only_query():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((90, D_QK)).astype(np.float32)
    qv = rng.standard_normal((2, D_QK)).astype(np.float32)
    qv[:, :D_V] = 0                         # scores depend on RoPE dims only
    q, kv, bt, sl = _single_request(keys, qv, 0.5)
    out1, lse1 = oracle.mla_decode(q, kv, bt, sl, 0.5)
    keys2 = keys.copy()
    keys2[:, :D_V] *= 4.0                   # power of two: exact in bf16
    q, kv, bt, sl = _single_request(keys2, qv, 0.5)
    out2, lse2 = oracle.mla_decode(q, kv, bt, sl, 0.5)
    assert np.allclose(out2, 4.0 * out1, rtol=1e-13, atol=1e-13)
    assert np.array_equal(lse1, lse2)


def test_naive_online_and_split_merge_agree():
    rng = np.random.default_rng(9)
    for L in (1, 5, 64, 100, 777):
        keys = rng.standard_normal((L, D_QK))
        qrows = rng.standard_normal((8, D_QK))
        o0, l0 = oracle.attend(qrows, keys, 0.07)
        for blk in (1, 7, 64):
            o1, l1 = oracle.online_attend(qrows, keys, 0.07, block=blk)
            assert np.allclose(o1, o0, rtol=0, atol=1e-12) and np.allclose(l1, l0, rtol=0, atol=1e-12)
        for _ in range(3):
            cuts = sorted(set(rng.integers(1, L, size=min(5, max(L - 1, 0))).tolist())) if L > 1 else []
            bounds = [0] + cuts + [L]
            o2, l2 = oracle.split_then_merge(qrows, keys, 0.07, bounds)
            assert np.allclose(o2, o0, rtol=0, atol=1e-12) and np.allclose(l2, l0, rtol=0, atol=1e-12)


def test_merge_skips_empty_splits():
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((50, D_QK))
    qrows = rng.standard_normal((3, D_QK))
    o0, l0 = oracle.attend(qrows, keys, 0.1)
    empty_o, empty_l = oracle.attend(qrows, keys[:0], 0.1)
    assert np.all(empty_o == 0) and np.all(np.isneginf(empty_l))
    o, l = oracle.merge_partials(np.stack([empty_o, o0, empty_o]), np.stack([empty_l, l0, empty_l]))
    assert np.allclose(o, o0, rtol=0, atol=1e-15) and np.allclose(l, l0, rtol=0, atol=1e-15)
    o, l = oracle.merge_partials(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_empty_request():
    inp = W.make_inputs(3, 1, 16, [0, 70, 0], pool=8, max_blocks=2, seed=4)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


def test_brute_force_exact_rational_tiny():
    """Exact rational dot products, then fsum-based softmax, on a tiny case."""
    inp = W.make_inputs(2, 2, 2, [3, 66], pool=6, max_blocks=2, seed=8)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale)
    scale = Fraction(inp.softmax_scale)
    for b in range(2):
        L = int(inp.cache_seqlens[b])
        toks = []
        for t in range(L):
            row = inp.kv_cache[inp.block_table[b, t // PAGE], t % PAGE, 0]
            toks.append([Fraction(float(x)) for x in W.bf16_bits_to_f32(row)])
        for s in range(2):
            for h in range(2):
                qq = [Fraction(float(x)) for x in W.bf16_bits_to_f32(inp.q[b, s, h])]
                sc = [float(scale * sum(a * c for a, c in zip(qq, k))) for k in toks]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                assert abs(lse[b, h, s] - (m + math.log(z))) < 1e-12
                for c in (0, 1, 255, 511):
                    ref = math.fsum(wi * float(k[c]) for wi, k in zip(w, toks)) / z
                    assert abs(out[b, s, h, c] - ref) < 1e-12


def test_rows_sampler_matches_full():
    inp = W.config_inputs(1)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale)
    picks = [(0, 0, 3), (1, 0, 15), (1, 0, 0)]
    o, l = oracle.mla_decode_rows(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                  inp.softmax_scale, picks)
    for k, (i, s, h) in enumerate(picks):
        # one row at a time vs a batched matmul: same math, BLAS may round differently
        assert np.allclose(o[k], out[i, s, h], rtol=0, atol=1e-13) and abs(l[k] - lse[i, h, s]) < 1e-13


def test_workload_recipe_properties():
    for idx in (1, 2):
        inp = W.config_inputs(idx)
        c = W.CONFIGS[idx]
        assert inp.q.shape == (c["batch"], c["s_q"], c["h_q"], D_QK)
        n = [(int(L) + 63) // 64 for L in inp.cache_seqlens]
        used = np.concatenate([inp.block_table[b, :n[b]] for b in range(inp.batch)])
        assert len(set(used.tolist())) == len(used)          # no page shared
        pad_pages = set(inp.block_table.ravel().tolist()) - set(used.tolist())
        for p in pad_pages:                                   # padding points at poison
            assert np.all(inp.kv_cache[p] == W.POISON_BITS)
    inp = W.config_inputs(1)
    assert list(inp.cache_seqlens) == [100, 257]
    assert inp.num_blocks == 16


# ---------------------------------------------------------------------------
# Causal masking for multi-token prediction (the API's is_causal flag): the
# s_q query tokens are the last s_q positions, token s sees keys
# 0 .. L - s_q + s.

@pytest.mark.parametrize("L", [1, 2, 3, 64, 65, 66, 130])
def test_causal_position_encoded_cache(L):
    """Uniform weights (scale 0) over position-encoded keys: token s of 3
    averages positions 0 .. L - 3 + s, so out = (L - 3 + s) / 2 and
    lse = ln(L - 2 + s); a token that sees no key gives 0 and -inf."""
    s_q = 3
    keys = np.zeros((L, D_QK), np.float32)
    keys[:, 0] = np.arange(L)
    q, kv, bt, sl = _single_request(keys, np.ones((s_q, D_QK), np.float32), 0.0, seed=L)
    q = q.reshape(1, s_q, 1, D_QK)
    out, lse = oracle.mla_decode(q, kv, bt, sl, 0.0, causal=True)
    for s in range(s_q):
        n = L - 2 + s            # keys 0 .. L - 3 + s
        if n <= 0:
            assert np.all(out[0, s, 0] == 0) and lse[0, 0, s] == -np.inf
        else:
            assert abs(out[0, s, 0, 0] - (n - 1) / 2) < 1e-12
            assert abs(lse[0, 0, s] - math.log(n)) < 1e-12


def test_causal_single_query_token_is_the_dense_result():
    inp = W.config_inputs(1)
    a = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale)
    b = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale, causal=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_brute_force_exact_rational_tiny():
    """Exact rational scores; token s of s_q = 2 keeps only keys t <= L - 2 + s."""
    inp = W.make_inputs(2, 2, 2, [2, 66], pool=6, max_blocks=2, seed=9)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale, causal=True)
    scale = Fraction(inp.softmax_scale)
    for b in range(2):
        L = int(inp.cache_seqlens[b])
        toks = []
        for t in range(L):
            row = inp.kv_cache[inp.block_table[b, t // PAGE], t % PAGE, 0]
            toks.append([Fraction(float(x)) for x in W.bf16_bits_to_f32(row)])
        for s in range(2):
            seen = [k for t, k in enumerate(toks) if t <= L - 2 + s]
            for h in range(2):
                qq = [Fraction(float(x)) for x in W.bf16_bits_to_f32(inp.q[b, s, h])]
                sc = [float(scale * sum(a * c for a, c in zip(qq, k))) for k in seen]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                assert abs(lse[b, h, s] - (m + math.log(z))) < 1e-12
                for c in (0, 3, 300, 511):
                    ref = math.fsum(wi * float(k[c]) for wi, k in zip(w, seen)) / z
                    assert abs(out[b, s, h, c] - ref) < 1e-12


def test_causal_rows_sampler_matches_full():
    inp = W.make_inputs(3, 2, 4, [70, 1, 129], pool=8, max_blocks=3, seed=10)
    out, lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                 inp.softmax_scale, causal=True)
    picks = [(0, 0, 1), (0, 1, 3), (1, 0, 0), (1, 1, 2), (2, 0, 3)]
    o, l = oracle.mla_decode_rows(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                  inp.softmax_scale, picks, causal=True)
    for k, (i, s, h) in enumerate(picks):
        if np.isneginf(lse[i, h, s]):
            assert np.isneginf(l[k]) and np.all(o[k] == 0)
        else:
            assert np.allclose(o[k], out[i, s, h], rtol=0, atol=1e-13) and abs(l[k] - lse[i, h, s]) < 1e-13


# ---------------------------------------------------------------------------
# Sparse (top-k) decode: pinned to the dense oracle through the identity
# gather, to closed forms under uniform weights (multiplicity, page/offset
# decoding), and to invariants (list order, padding, truncation).

def _dense_as_sparse(inp, topk, pad_value=-1):
    """Index lists naming each request's dense keys in logical order,
    padded with ``pad_value`` up to ``topk`` (page_id * 64 + offset)."""
    b, s_q = inp.batch, inp.s_q
    idx = np.full((b, s_q, topk), pad_value, dtype=np.int32)
    for i in range(b):
        L = int(inp.cache_seqlens[i])
        t = np.arange(L)
        phys = inp.block_table[i, t // PAGE].astype(np.int64) * PAGE + t % PAGE
        idx[i, :, :L] = phys
    return idx


def test_sparse_identity_gather_equals_dense():
    inp = W.make_inputs(3, 2, 4, [100, 257, 64], pool=12, max_blocks=6, seed=5)
    idx = _dense_as_sparse(inp, 300)
    o_d, l_d = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale)
    o_s, l_s = oracle.mla_decode_sparse(inp.q, inp.kv_cache, idx, inp.softmax_scale)
    assert np.allclose(o_s, o_d, rtol=0, atol=1e-12) and np.allclose(l_s, l_d, rtol=0, atol=1e-12)
    # The same lists without padding, cut by topk_length instead.
    idx2 = _dense_as_sparse(inp, 300, pad_value=0)
    o_t, l_t = oracle.mla_decode_sparse(inp.q, inp.kv_cache, idx2[:, :, :257], inp.softmax_scale,
                                        topk_length=inp.cache_seqlens)
    assert np.allclose(o_t, o_d, rtol=0, atol=1e-12) and np.allclose(l_t, l_d, rtol=0, atol=1e-12)


def test_sparse_index_decodes_page_and_offset():
    """Row r of block p holds V = (p, r, 1, 0, ...) and K = 0: with uniform
    weights out is the mean of the named (page, offset) pairs, so a swapped
    page/offset decoding or a wrong block stride shows directly."""
    pool = 5
    kv = np.zeros((pool, PAGE, 1, D_QK), dtype=np.uint16)
    for p in range(pool):
        for r in range(PAGE):
            kv[p, r, 0, :3] = _bits([p, r, 1.0])
    q = _bits(np.zeros((1, 1, 1, D_QK), np.float32))
    picks = [(3, 7), (0, 63), (4, 0), (1, 32)]
    idx = np.array([[[p * PAGE + r for p, r in picks]]], dtype=np.int32)
    out, lse = oracle.mla_decode_sparse(q, kv, idx, 0.5)
    assert out[0, 0, 0, 0] == pytest.approx(np.mean([p for p, _ in picks]), abs=1e-12)
    assert out[0, 0, 0, 1] == pytest.approx(np.mean([r for _, r in picks]), abs=1e-12)
    assert out[0, 0, 0, 2] == pytest.approx(1.0, abs=1e-12)
    assert lse[0, 0, 0] == pytest.approx(math.log(len(picks)), abs=1e-12)


def test_sparse_list_is_a_multiset():
    """softmax_scale = 0: every listed entry weighs the same, so an index
    named twice counts twice (out = (2 V_a + V_b) / 3, lse = ln 3)."""
    rng = np.random.default_rng(11)
    kv = _bits(rng.standard_normal((2, PAGE, 1, D_QK)).astype(np.float32))
    q = _bits(rng.standard_normal((1, 1, 2, D_QK)).astype(np.float32))
    a, b = 70, 5
    idx = np.array([[[a, b, a]]], dtype=np.int32)
    out, lse = oracle.mla_decode_sparse(q, kv, idx, 0.0)
    rows = oracle.bf16_to_f64(kv.reshape(-1, D_QK))
    want = (2 * rows[a, :D_V] + rows[b, :D_V]) / 3
    assert np.allclose(out[0, 0], want[None, :], rtol=0, atol=1e-12)
    assert np.allclose(lse[0, :, 0], math.log(3), rtol=0, atol=1e-12)


def test_sparse_padding_order_and_truncation():
    inp = W.make_sparse_inputs(2, 2, 3, 40, [200, 130], seed=3, pad_frac=0.25)
    o, l = oracle.mla_decode_sparse(inp.q, inp.kv_cache, inp.indices, inp.softmax_scale)
    # Order of the list does not matter (padding included).
    rng = np.random.default_rng(0)
    shuf = inp.indices.copy()
    for i in range(2):
        for s in range(2):
            shuf[i, s] = shuf[i, s, rng.permutation(40)]
    o2, l2 = oracle.mla_decode_sparse(inp.q, inp.kv_cache, shuf, inp.softmax_scale)
    assert np.allclose(o2, o, rtol=0, atol=1e-12) and np.allclose(l2, l, rtol=0, atol=1e-12)
    # Padding entries (-1) and entries past the pool name no key: the same as dropping them.
    big = inp.indices.copy()
    big[big < 0] = inp.kv_cache.shape[0] * PAGE + 17
    o3, l3 = oracle.mla_decode_sparse(inp.q, inp.kv_cache, big, inp.softmax_scale)
    assert np.allclose(o3, o, rtol=0, atol=1e-12) and np.allclose(l3, l, rtol=0, atol=1e-12)
    i, s = 1, 0
    kept = inp.indices[i, s][inp.indices[i, s] >= 0]
    o4, l4 = oracle.mla_decode_sparse(inp.q[i:i + 1, s:s + 1], inp.kv_cache, kept[None, None, :], inp.softmax_scale)
    assert np.allclose(o4[0, 0], o[i, s], rtol=0, atol=1e-12) and np.allclose(l4[0, :, 0], l[i, :, s], atol=1e-12)
    # topk_length keeps the first entries of each list of that request.
    o5, l5 = oracle.mla_decode_sparse(inp.q, inp.kv_cache, inp.indices, inp.softmax_scale, topk_length=[40, 25])
    o6, l6 = oracle.mla_decode_sparse(inp.q[1:], inp.kv_cache, inp.indices[1:, :, :25], inp.softmax_scale)
    assert np.allclose(o5[0], o[0], atol=1e-12) and np.allclose(o5[1], o6[0], atol=1e-12)
    assert np.allclose(l5[1], l6[0], atol=1e-12)


def test_sparse_no_key_gives_zero_and_minus_inf():
    inp = W.make_sparse_inputs(2, 1, 4, 8, [64, 64], seed=2)
    idx = inp.indices.copy()
    idx[0] = -1
    out, lse = oracle.mla_decode_sparse(inp.q, inp.kv_cache, idx, inp.softmax_scale, topk_length=[8, 0])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------------------
# FP8 cache records: the e4m3 code points of the OCP format, the record
# layout (latent | 4 fp32 scales | bf16 RoPE), per-tile scales, and the
# fp32-then-bf16 rounding of the dequantized value, all against hand values.

def test_e4m3_code_points():
    ocp = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
           0x40: 2.0, 0x7e: 448.0, 0xc0: -2.0, 0xb8: -1.0, 0xfe: -448.0}
    for b, v in ocp.items():
        assert oracle.e4m3_value(b) == v, hex(b)
    assert math.isnan(oracle.e4m3_value(0x7f)) and math.isnan(oracle.e4m3_value(0xff))
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0 and oracle.e4m3_value(0x80) == 0.0
    vals = [oracle.e4m3_value(b) for b in range(0x7f)]
    assert all(a < b for a, b in zip(vals, vals[1:]))                       # 0x00..0x7e ascending
    assert all(oracle.e4m3_value(b | 0x80) == -oracle.e4m3_value(b) for b in range(1, 0x7f))


def _record(lat_bytes, scales, rope_bits):
    rec = np.zeros((1, PAGE, 1, 656), np.uint8)
    rec[0, :, 0, :512] = np.asarray(lat_bytes, np.uint8)
    rec[0, :, 0, 512:528] = np.asarray(scales, np.float32).view(np.uint8)
    rec[0, :, 0, 528:] = np.asarray(rope_bits, np.uint16).view(np.uint8)
    return rec


def test_fp8_record_layout_and_tile_scales():
    rope = (np.arange(64, dtype=np.uint16) + 0x3F00)        # distinct bf16 patterns
    k = oracle.dequantize_fp8_cache(_record(np.full(512, 0x38), [0.5, 2.0, 3.0, 1e-3], rope))
    assert k.shape == (1, PAGE, 1, D_QK)
    row = k[0, 5, 0]
    assert np.all(row[0:128] == 0x3F00)       # 1.0 * 0.5
    assert np.all(row[128:256] == 0x4000)     # 1.0 * 2
    assert np.all(row[256:384] == 0x4040)     # 1.0 * 3
    assert np.all(row[384:512] == 0x3A83)     # fp32(1e-3) = 0x3A83126F -> bf16 0x3A83
    assert np.array_equal(row[512:], rope)    # RoPE copied, not scaled


def test_fp8_dequantize_rounds_to_fp32_then_bf16_nearest_even():
    # 1.125 * 1.0078125 = 1.1337890625 = 1 + 17.125/128 -> bf16 1 + 17/128 = 1.1328125 (0x3F91)
    # 1.0 * (1 + 2^-8) is a tie between 1 and 1 + 2^-7: even mantissa, 1.0 (0x3F80)
    # 1.0 * (1 + 3 * 2^-8) is a tie between 1 + 2^-7 and 1 + 2^-6: even, 1 + 2^-6 (0x3F82)
    # 2^-9 * 2^-126 = 2^-135: an fp32 subnormal, below half of the smallest bf16 one (2^-133), so 0
    lat = np.array([0x39] * 128 + [0x38] * 128 + [0x38] * 128 + [0x01] * 128)
    k = oracle.dequantize_fp8_cache(_record(lat, [1.0078125, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2.0 ** -126],
                                            np.zeros(64)))
    row = k[0, 0, 0]
    assert np.all(row[0:128] == 0x3F91) and np.all(row[128:256] == 0x3F80)
    assert np.all(row[256:384] == 0x3F82) and np.all(row[384:512] == 0x0000)


def test_fp8_records_round_trip_within_e4m3_precision():
    inp = W.make_inputs(1, 1, 16, [128], pool=3, max_blocks=2, seed=8)
    kv = inp.kv_cache[inp.block_table[0, :2]]
    back = W.bf16_bits_to_f32(oracle.dequantize_fp8_cache(W.to_fp8_records(kv))).astype(np.float64)
    x = W.bf16_bits_to_f32(kv).astype(np.float64)
    # e4m3 keeps 4 significant bits: |error| <= 2^-4 |x| + (subnormal step) * scale, plus bf16 rounding.
    amax = np.abs(x[..., :512]).reshape(2, PAGE, 1, 4, 128).max(-1, keepdims=True)
    step = np.broadcast_to(amax / 448 * 2.0 ** -9, (2, PAGE, 1, 4, 128)).reshape(2, PAGE, 1, 512)
    err = np.abs(back - x)[..., :512]
    assert np.all(err <= 2.0 ** -4 * np.abs(x[..., :512]) + step + 2.0 ** -8 * np.abs(x[..., :512]))
    assert np.array_equal(back[..., 512:], x[..., 512:])
