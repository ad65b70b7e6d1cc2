"""GPU parity tests of the FP8 cache (656-byte records: e4m3 latent, four
fp32 tile scales, bf16 RoPE) through the C ABI, dense and sparse, against
the oracle on the dequantized cache: a single key per request (the output is
then the dequantized V row itself, so the in-kernel dequantization is checked
bit for bit), every kernel (16 rows; 128-row groups, one or two; 32 and 64
rows on the 128-row kernel), ragged lengths, forced splits, the causal mask,
NaN records past the sequence end, and the memory-bound workload in full."""
import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, out_tol_bound

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda", 0))


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.device("cuda", 0))


def run_dense_fp8(inp, rec, force_splits=0, num_cus=0, causal=False):
    import torch
    print(f"[fp8] dense b={inp.batch} s_q={inp.s_q} h_q={inp.h_q} force={force_splits} causal={causal}", flush=True)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, num_cus=num_cus, force_splits=force_splits)
    out, lse = mla.mla_decode_fwd(_bf16(inp.q), _dev(rec), _dev(inp.block_table), _dev(inp.cache_seqlens),
                                  inp.softmax_scale, sched, ns, causal=causal, fp8=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref_dense_fp8(inp, rec, causal=False):
    kv = oracle.dequantize_fp8_cache(rec)
    return oracle.mla_decode(inp.q, kv, inp.block_table, inp.cache_seqlens, inp.softmax_scale, causal=causal)


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_single_key_output_is_the_dequantized_row(h_q):
    inp = W.make_inputs(3, 1, h_q, [1, 1, 1], pool=6, max_blocks=2, seed=31)
    rec = W.to_fp8_records(inp.kv_cache)
    out, lse = run_dense_fp8(inp, rec)
    kv = oracle.dequantize_fp8_cache(rec)
    for i in range(3):
        v = W.bf16_bits_to_f32(kv[inp.block_table[i, 0], 0, 0, :512]).astype(np.float64)
        assert np.array_equal(out[i, 0], np.broadcast_to(v, out[i, 0].shape)), f"request {i}"
    ref_out, ref_lse = ref_dense_fp8(inp, rec)
    assert_parity(out, lse, ref_out, ref_lse, f"fp8 single key h_q={h_q}")


CASES = [
    # h_q, s_q, lengths, force_splits, causal
    (16, 1, [100, 257, 1, 640], 0, False),
    (16, 1, [1000, 2000], 3, False),
    (16, 2, [70, 300], 0, True),
    (128, 1, [64, 300, 1100], 0, False),
    (128, 2, [129, 700], 2, True),
    (64, 1, [200, 900], 0, False),
    (32, 2, [90, 600], 2, False),
    (256, 1, [300, 65], 0, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_dense_parity(case):
    h_q, s_q, lens, force, causal = CASES[case]
    inp = W.make_inputs(len(lens), s_q, h_q, lens, pool=None, max_blocks=max(-(-L // 64) for L in lens) + 1,
                        seed=50 + case)
    rec = W.to_fp8_records(inp.kv_cache)
    ref_out, ref_lse = ref_dense_fp8(inp, rec, causal=causal)
    out, lse = run_dense_fp8(inp, rec, force_splits=force, causal=causal)
    assert_parity(out, lse, ref_out, ref_lse, f"fp8 dense case {case}", out_tol=out_tol_bound(inp))


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_nan_records_past_the_end_do_not_leak(h_q):
    inp = W.make_inputs(2, 1, h_q, [100, 193], pool=8, max_blocks=4, seed=33)
    rec = W.to_fp8_records(inp.kv_cache)
    for i, L in enumerate(inp.cache_seqlens):
        last = inp.block_table[i, (L - 1) // 64]
        rec[last, L % 64 or 64:, 0, :] = 0x7F            # e4m3 NaN bytes, NaN scales and RoPE
    used = set(int(x) for i, L in enumerate(inp.cache_seqlens) for x in inp.block_table[i, :-(-L // 64)])
    for pg in range(rec.shape[0]):
        if pg not in used:
            rec[pg] = 0x7F
    ref_out, ref_lse = ref_dense_fp8(inp, rec)
    assert np.isfinite(ref_out).all()
    for force in (0, 2):
        out, lse = run_dense_fp8(inp, rec, force_splits=force)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        assert_parity(out, lse, ref_out, ref_lse, f"fp8 NaN tails h_q={h_q} force={force}",
                      out_tol=out_tol_bound(inp))


def test_fp8_memory_bound_workload_full():
    inp = W.config_inputs(2)
    rec = W.to_fp8_records(inp.kv_cache)
    ref_out, ref_lse = ref_dense_fp8(inp, rec)
    out, lse = run_dense_fp8(inp, rec)
    assert_parity(out, lse, ref_out, ref_lse, "fp8 memory-bound workload")


def run_sparse_fp8(inp, rec, num_cus=0):
    import torch
    b, s_q, topk = inp.indices.shape
    print(f"[fp8] sparse b={b} s_q={s_q} h_q={inp.h_q} topk={topk} num_cus={num_cus}", flush=True)
    sched, ns = mla.get_mla_metadata_sparse(inp.topk_length, b, s_q, inp.h_q, topk, num_cus=num_cus)
    tl = None if inp.topk_length is None else _dev(np.asarray(inp.topk_length, np.int32))
    out, lse = mla.mla_decode_sparse_fwd(_bf16(inp.q), _dev(rec), _dev(inp.indices), inp.softmax_scale, sched, ns,
                                         topk_length=tl, fp8=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


SPARSE_CASES = [
    # h_q, s_q, topk, context, pad_frac, topk_length, num_cus
    (16, 2, 200, [300, 500, 1000], 0.1, [200, 150, 1], 256),
    (16, 1, 64, [64, 128], 0.0, None, 0),
    (128, 2, 333, [400, 700, 333], 0.2, [333, 100, 0], 0),
    (128, 1, 1, [64, 70], 0.0, None, 16),
    (64, 1, 700, [800, 900], 0.0, None, 0),
]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
def test_fp8_sparse_parity(case):
    from test_sparse_gpu import sparse_out_tol
    h_q, s_q, topk, ctx, pad, tl, cus = SPARSE_CASES[case]
    inp = W.make_sparse_inputs(len(ctx), s_q, h_q, topk, ctx, seed=70 + case, pad_frac=pad, topk_length=tl)
    rec = W.to_fp8_records(inp.kv_cache)
    kv = oracle.dequantize_fp8_cache(rec)
    ref_out, ref_lse = oracle.mla_decode_sparse(inp.q, kv, inp.indices, inp.softmax_scale, topk_length=inp.topk_length)
    out, lse = run_sparse_fp8(inp, rec, num_cus=cus)
    deq = W.SparseInputs(inp.name, inp.q, kv, inp.indices, inp.topk_length, inp.softmax_scale)
    assert_parity(out, lse, ref_out, ref_lse, f"fp8 sparse case {case}", out_tol=sparse_out_tol(deq))
