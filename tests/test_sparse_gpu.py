"""GPU parity tests of sparse (top-k) decode through the C ABI
(mla_get_metadata_sparse + mla_decode_sparse_fwd) against the CPU oracle:
gathered copies from per-token indices, -1 padding and out-of-range entries,
topk_length, ragged list lengths, split pieces, every kernel the sparse path
uses (h_q <= 16 in one workgroup; 128-row workgroups above, one or two row
groups, R below 128), a query token with no key, the restart path, and the
identity gather against the dense path bit for bit."""
import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, max_err, sparse_out_bound, to_device

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.device("cuda", 0)) if dtype is None else t.to(torch.device("cuda", 0), dtype)


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.device("cuda", 0))


def run_sparse(inp, num_cus=0, indices=None, topk_length="inp"):
    import torch
    idx = inp.indices if indices is None else indices
    tl = inp.topk_length if isinstance(topk_length, str) else topk_length
    b, s_q, topk = idx.shape
    print(f"[sparse] b={b} s_q={s_q} h_q={inp.h_q} topk={topk} topk_length={'none' if tl is None else 'set'} "
          f"num_cus={num_cus}", flush=True)
    sched, ns = mla.get_mla_metadata_sparse(tl, b, s_q, inp.h_q, topk, num_cus=num_cus)
    out, lse = mla.mla_decode_sparse_fwd(_bf16(inp.q), _bf16(inp.kv_cache), _dev(idx), inp.softmax_scale, sched, ns,
                                         topk_length=None if tl is None else _dev(np.asarray(tl, np.int32)))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _ref(inp, indices=None, topk_length="inp"):
    idx = inp.indices if indices is None else indices
    tl = inp.topk_length if isinstance(topk_length, str) else topk_length
    return oracle.mla_decode_sparse(inp.q, inp.kv_cache, idx, inp.softmax_scale, topk_length=tl)


CASES = [
    # h_q, s_q, topk, context, pad_frac, topk_length, num_cus
    (16, 1, 64, [64, 128, 300], 0.0, None, 0),
    (16, 2, 200, [300, 500, 1000], 0.1, [200, 150, 1], 256),
    (16, 3, 1000, [1000, 1500], 0.0, [700, 1000], 0),
    (8, 1, 130, [200, 200, 260, 1300], 0.05, None, 64),
    (128, 1, 512, [600, 2000], 0.0, None, 256),
    (128, 2, 333, [400, 700, 333], 0.2, [333, 100, 0], 0),
    (64, 2, 256, [256, 1000], 0.0, None, 0),
    (32, 1, 1, [64, 70], 0.0, None, 16),
    (256, 1, 300, [300, 900], 0.1, None, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sparse_parity(case):
    h_q, s_q, topk, ctx, pad, tl, cus = CASES[case]
    inp = W.make_sparse_inputs(len(ctx), s_q, h_q, topk, ctx, seed=40 + case, pad_frac=pad, topk_length=tl)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_sparse(inp, num_cus=cus)
    assert_parity(out, lse, ref_out, ref_lse, f"sparse case {case}", out_tol=sparse_out_bound(inp))


@pytest.mark.parametrize("h_q", [16, 128])
def test_sparse_degenerate_lists(h_q):
    """A token with no key (all padding, or topk_length 0), entries past the
    pool, duplicates, and lists whose valid entries are scattered."""
    inp = W.make_sparse_inputs(3, 2, h_q, 150, [300, 300, 300], seed=7)
    idx = inp.indices.copy()
    idx[0, 0] = -1                                        # query with no key
    idx[0, 1, ::2] = inp.kv_cache.shape[0] * 64 + 5      # past the pool: no key
    idx[1, 0, 10:40] = idx[1, 0, 0]                      # one row named 31 times
    idx[1, 1, 64:128] = -1                               # a whole padded page in the middle
    idx[2, 1, :] = idx[2, 1, ::-1]
    tl = [150, 150, 0]                                   # request 2 sees nothing
    ref_out, ref_lse = _ref(inp, idx, tl)
    assert np.isneginf(ref_lse[0, :, 0]).all() and np.isneginf(ref_lse[2]).all()
    for cus in (0, 256):
        out, lse = run_sparse(inp, num_cus=cus, indices=idx, topk_length=tl)
        assert_parity(out, lse, ref_out, ref_lse, f"degenerate lists h_q={h_q} cus={cus}",
                      out_tol=sparse_out_bound(inp, idx, tl))
        assert np.all(out[0, 0] == 0) and np.all(out[2] == 0)


@pytest.mark.parametrize("h_q", [16, 128])
def test_sparse_identity_gather_equals_dense_bitwise(h_q):
    """Index lists naming each request's dense keys in order: same plan, same
    pages, same arithmetic as the dense path, so the outputs agree bit for bit."""
    import torch
    inp = W.make_inputs(4, 1, h_q, [70, 640, 1, 3000], pool=70, max_blocks=48, seed=9)
    topk = 3008
    idx = np.full((4, 1, topk), -1, dtype=np.int32)
    for i in range(4):
        L = int(inp.cache_seqlens[i])
        t = np.arange(L)
        idx[i, 0, :L] = inp.block_table[i, t // 64] * 64 + t % 64
    d = to_device(inp)
    for cus in (0, 256):
        hs, hn = mla.get_mla_metadata(inp.cache_seqlens, h_q, 1, num_cus=cus)
        dense_o, dense_l = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, hs, hn)
        ss, sn = mla.get_mla_metadata_sparse(inp.cache_seqlens, 4, 1, h_q, topk, num_cus=cus)
        assert torch.equal(ss.cpu(), hs.cpu()) and torch.equal(sn.cpu(), hn.cpu())
        sp_o, sp_l = mla.mla_decode_sparse_fwd(d["q"], d["kv"], _dev(idx), inp.softmax_scale, ss, sn,
                                               topk_length=d["sl"])
        torch.cuda.synchronize()
        print(f"[sparse] identity gather h_q={h_q} cus={cus}", flush=True)
        assert torch.equal(sp_o, dense_o) and torch.equal(sp_l, dense_l)


@pytest.mark.parametrize("h_q", [16, 128])
def test_sparse_restart_when_later_page_outgrows_first_max(h_q):
    rng = np.random.default_rng(4)
    inp = W.make_sparse_inputs(1, 1, h_q, 64 * 4 + 9, [900], seed=13)
    rows = inp.kv_cache.reshape(-1, W.D_QK)
    keys = (0.01 * rng.standard_normal((inp.topk, W.D_QK))).astype(np.float32)
    keys[64 * 2 + 3] = 0.5      # listed on page 2: far above page 0's maximum
    keys[64 * 3 + 1] = -0.5
    for i, e in enumerate(inp.indices[0, 0]):
        rows[e] = W.f32_to_bf16_bits(keys[i])
    q = np.abs(rng.standard_normal((1, 1, h_q, W.D_QK))).astype(np.float32)
    if h_q >= 128:
        q[0, 0, :32] *= 1e-3
        q[0, 0, 64:] *= 1e-3
    inp.q = W.f32_to_bf16_bits(q)
    inp.softmax_scale = 1.0
    ref_out, ref_lse = _ref(inp)
    assert ref_lse.max() > 100
    for cus in (0, 256):
        out, lse = run_sparse(inp, num_cus=cus)
        assert_parity(out, lse, ref_out, ref_lse, f"sparse restart h_q={h_q} cus={cus}", out_tol=sparse_out_bound(inp))


def test_sparse_workload_full():
    """The sparse workload (batch 128, s_q 2, h_q 128, topk 2048) in the launch
    configuration the benchmark times, every output against the oracle."""
    inp = W.sparse_config_inputs()
    out, lse = run_sparse(inp)
    ref_out, ref_lse = _ref(inp)
    assert_parity(out, lse, ref_out, ref_lse, "sparse workload (full)")


@pytest.mark.parametrize("cus", [0, 256])
def test_sparse_scale_zero_with_padded_page_starts(cus):
    """softmax_scale = 0 (uniform weights over the listed keys) with the first
    32 entries of every 64-entry page padded (-1), so every piece, wherever the
    plan starts it, begins with a 32-token tile that has no key: the 128-row
    kernel's first tile then has max -inf, and -inf * 0 must not become its
    reference (out = the mean of the listed V rows, lse = ln(count))."""
    inp = W.make_sparse_inputs(3, 2, 128, 640, [700, 900, 1300], seed=17)
    idx = inp.indices.copy()
    for pg in range(0, 640, 64):
        idx[:, :, pg:pg + 32] = -1
    inp.softmax_scale = 0.0
    ref_out, ref_lse = _ref(inp, idx, None)
    out, lse = run_sparse(inp, num_cus=cus, indices=idx, topk_length=None)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert_parity(out, lse, ref_out, ref_lse, f"sparse scale 0, padded page starts, cus={cus}",
                  out_tol=sparse_out_bound(inp, idx, None))
    assert max_err(lse, np.full_like(lse, np.log(320.0))) <= 1e-3
