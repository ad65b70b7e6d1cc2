"""CPU check of the elementwise output bound the GPU parity tests use
(``gpu_util.row_out_bound``): an emulation of the HIP path's rounding steps
(fp32 scores, base-2 exponentials against a fixed reference, bf16
probabilities with an fp32 row sum, split pieces merged through fp32
partials, bf16 output) stays inside the bound, and plausible mistakes (a
dropped key, a wrong score scale, a sign error in one output column, a
partial merged with the wrong weight) do not.  (Summing the bf16-rounded
probabilities instead of the fp32 ones is an error of the bound's own size,
not a mistake it can tell apart.)
Both sides use the oracle's gather of the keys; no GPU is involved."""
import numpy as np
import pytest

import oracle
from decode_attention_mla_amd import workloads as W
from gpu_util import U_BF16, row_out_bound

LOG2E = np.float32(1.4426950408889634)


def _bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(x, np.float32)))


def emulate(q, keys, scale, pieces=1, mistake=None):
    """The kernel's arithmetic on one request: q float32 [R, 576], keys
    float32 [L, 576] (bf16 values).  Each piece keeps its first page's row max
    as the reference, exponentiates in base 2, rounds P to bf16 for PV and sums
    the fp32 values; pieces are merged by their base-2 lse; out is bf16."""
    L = keys.shape[0]
    sl = np.float32(scale) * LOG2E
    if mistake == "scale":
        sl = sl * np.float32(1.05)
    if mistake == "drop":
        keys = np.delete(keys, L // 2, axis=0)
        L -= 1
    bounds = np.linspace(0, L, pieces + 1).astype(int)
    parts_o, parts_l = [], []
    for a, e in zip(bounds[:-1], bounds[1:]):
        s = (q @ keys[a:e].T).astype(np.float32) * sl                   # fp32 scores, base 2
        m_ref = s[:, :min(64, e - a)].max(axis=1, keepdims=True)
        p = np.exp2(s - m_ref).astype(np.float32)
        pb = _bf16(p)
        l = p.sum(axis=1, dtype=np.float32)
        o = (pb @ keys[a:e, :512]).astype(np.float32) / l[:, None]
        parts_o.append(o)
        parts_l.append(m_ref[:, 0] + np.log2(l).astype(np.float32))
    M = np.max(parts_l, axis=0)
    w = [np.exp2(lv - M).astype(np.float32) for lv in parts_l]
    if mistake == "merge" and pieces > 1:
        w[0] = w[0] * np.float32(1.1)
    acc = sum(wi[:, None] * oi for wi, oi in zip(w, parts_o))
    out = _bf16(acc / sum(w)[:, None])
    if mistake == "sign":
        out[:, 7] = -out[:, 7]
    return out


def _case(seed, L, R=16, scale=W.SOFTMAX_SCALE, spread=1.0):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((R, 576)).astype(np.float32) * spread)
    k = _bf16(rng.standard_normal((L, 576)).astype(np.float32))
    return q, k, scale


@pytest.mark.parametrize("seed,L,pieces,spread", [(0, 1, 1, 1.0), (1, 7, 1, 1.0), (2, 300, 1, 1.0),
                                                  (3, 1000, 4, 1.0), (4, 2500, 9, 1.0), (5, 200, 2, 3.0),
                                                  (6, 64, 1, 6.0)])
def test_emulated_kernel_arithmetic_stays_inside_the_bound(seed, L, pieces, spread):
    q, k, scale = _case(seed, L, spread=spread)
    ref, _ = oracle.attend(q.astype(np.float64), k.astype(np.float64), scale)
    got = emulate(q, k, scale, pieces=pieces)
    tol = row_out_bound(q.astype(np.float64), k.astype(np.float64), scale)
    err = np.abs(got - ref)
    print(f"L={L} pieces={pieces} max err {err.max():.3e} worst err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("mistake", ["drop", "scale", "sign", "merge"])
def test_planted_mistakes_break_the_bound(mistake):
    q, k, scale = _case(11, 700, spread=2.0)
    ref, _ = oracle.attend(q.astype(np.float64), k.astype(np.float64), scale)
    tol = row_out_bound(q.astype(np.float64), k.astype(np.float64), scale)
    got = emulate(q, k, scale, pieces=3, mistake=mistake)
    assert np.any(np.abs(got - ref) > tol), mistake


def test_bound_is_at_least_the_output_rounding():
    # A single key: weight 1, out = v exactly; the bound is the bf16 half-ulp scale.
    q, k, scale = _case(21, 1)
    tol = row_out_bound(q.astype(np.float64), k.astype(np.float64), scale)
    v = np.abs(k[0, :512].astype(np.float64))
    assert np.all(tol >= U_BF16 * v) and np.all(tol <= 3 * U_BF16 * v + 1e-6)
