"""GPU parity tests of the FP8 cache (656-byte records: e4m3 latent, four
fp32 tile scales, bf16 RoPE) through the C ABI, dense and sparse, against
the oracle on the dequantized cache: a single key per request (the output is
then the dequantized V row itself, so the in-kernel dequantization is checked
bit for bit), every kernel (16 rows; 128-row groups, one or two; 32 and 64
rows on the 128-row kernel), ragged lengths, forced splits, the causal mask,
NaN records past the sequence end, the restart path, sparse identity lists
against the dense path bit for bit, graph replay, and the memory-bound
workload in full."""
import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, sparse_out_bound

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
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, num_cus=num_cus, force_splits=force_splits,
                                      fp8=True)
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
    assert_parity(out, lse, ref_out, ref_lse, f"fp8 dense case {case}",
                  out_tol=dense_out_bound(inp, causal=causal, kv=oracle.dequantize_fp8_cache(rec)))


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
                      out_tol=dense_out_bound(inp, kv=oracle.dequantize_fp8_cache(rec)))


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
    h_q, s_q, topk, ctx, pad, tl, cus = SPARSE_CASES[case]
    inp = W.make_sparse_inputs(len(ctx), s_q, h_q, topk, ctx, seed=70 + case, pad_frac=pad, topk_length=tl)
    rec = W.to_fp8_records(inp.kv_cache)
    kv = oracle.dequantize_fp8_cache(rec)
    ref_out, ref_lse = oracle.mla_decode_sparse(inp.q, kv, inp.indices, inp.softmax_scale, topk_length=inp.topk_length)
    out, lse = run_sparse_fp8(inp, rec, num_cus=cus)
    assert_parity(out, lse, ref_out, ref_lse, f"fp8 sparse case {case}", out_tol=sparse_out_bound(inp, kv=kv))


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_restart_when_later_page_outgrows_first_max(h_q):
    """First page scores ~0, a later page's ~+150 (far beyond the 2^64
    headroom of the first page's reference): the restart path of the FP8
    kernels (records read a page ahead on the small kernel) must match."""
    rng = np.random.default_rng(3)
    L = 64 * 5 + 7
    keys = (0.01 * rng.standard_normal((L, W.D_QK))).astype(np.float32)
    keys[64 * 3 + 5, :] = 0.5
    keys[64 * 4 + 1, :] = -0.5
    q = np.abs(rng.standard_normal((1, 1, h_q, W.D_QK))).astype(np.float32)
    if h_q >= 128:
        keep = np.zeros(h_q, dtype=bool)
        keep[32:64] = True
        q[0, 0, ~keep] *= 1e-3
    inp = W.make_inputs(1, 1, h_q, [L], pool=8, max_blocks=6, seed=5)
    kv = inp.kv_cache.copy()
    for t in range(L):
        kv[inp.block_table[0, t // 64], t % 64, 0] = W.f32_to_bf16_bits(keys[t])
    inp.kv_cache = kv
    inp.q = W.f32_to_bf16_bits(q)
    inp.softmax_scale = 1.0
    rec = W.to_fp8_records(inp.kv_cache)
    ref_out, ref_lse = ref_dense_fp8(inp, rec)
    assert ref_lse.max() > 100
    tol = dense_out_bound(inp, kv=oracle.dequantize_fp8_cache(rec))
    for force in (0, 1):
        out, lse = run_dense_fp8(inp, rec, force_splits=force)
        assert_parity(out, lse, ref_out, ref_lse, f"fp8 restart h_q={h_q} force={force}", out_tol=tol)


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_sparse_identity_gather_equals_dense_bitwise(h_q):
    """Index lists naming each request's dense keys in order, on FP8
    records: the sparse kernels (gathered records, key masks) and the dense
    ones (block-table records, read a page ahead on the small kernel) run
    the same plan and the same arithmetic, so they agree bit for bit."""
    import torch
    inp = W.make_inputs(4, 1, h_q, [70, 640, 1, 3000], pool=70, max_blocks=48, seed=9)
    rec = W.to_fp8_records(inp.kv_cache)
    topk = 3008
    idx = np.full((4, 1, topk), -1, dtype=np.int32)
    for i in range(4):
        L = int(inp.cache_seqlens[i])
        t = np.arange(L)
        idx[i, 0, :L] = inp.block_table[i, t // 64] * 64 + t % 64
    q, kv = _bf16(inp.q), _dev(rec)
    bt, sl = _dev(inp.block_table), _dev(inp.cache_seqlens)
    for cus in (0, 256):
        print(f"[fp8] identity gather h_q={h_q} cus={cus}", flush=True)
        hs, hn = mla.get_mla_metadata(inp.cache_seqlens, h_q, 1, num_cus=cus, fp8=True)
        dense_o, dense_l = mla.mla_decode_fwd(q, kv, bt, sl, inp.softmax_scale, hs, hn, fp8=True)
        ss, sn = mla.get_mla_metadata_sparse(inp.cache_seqlens, 4, 1, h_q, topk, num_cus=cus)
        assert torch.equal(ss.cpu(), hs.cpu()) and torch.equal(sn.cpu(), hn.cpu())
        sp_o, sp_l = mla.mla_decode_sparse_fwd(q, kv, _dev(idx), inp.softmax_scale, ss, sn, topk_length=sl, fp8=True)
        torch.cuda.synchronize()
        assert torch.equal(sp_o, dense_o) and torch.equal(sp_l, dense_l)


def test_fp8_graph_replay_matches_eager():
    """The memory-bound workload on FP8 records, one decode call captured in
    a HIP graph and replayed with eager work between replays: every replay
    reproduces the eager result bit for bit."""
    import torch
    inp = W.config_inputs(2)
    rec = W.to_fp8_records(inp.kv_cache)
    q, kv = _bf16(inp.q), _dev(rec)
    bt, sl = _dev(inp.block_table), _dev(inp.cache_seqlens)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, fp8=True)
    ref_out, ref_lse = mla.mla_decode_fwd(q, kv, bt, sl, inp.softmax_scale, sched, ns, fp8=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
    out, lse = torch.empty_like(ref_out), torch.empty_like(ref_lse)
    ws = torch.empty(mla.mla_workspace_bytes(sched.shape[0] + inp.batch - 1, inp.h_q, inp.s_q),
                     dtype=torch.uint8, device=out.device)

    def call():
        mla.mla_decode_fwd(q, kv, bt, sl, inp.softmax_scale, sched, ns, out=out, lse=lse, workspace=ws, fp8=True)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    print("[fp8] graph replay", flush=True)
    for _ in range(4):
        out.zero_()
        lse.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_records_beyond_4_gib_of_pool(h_q):
    """FP8 records at byte offsets past 2^32 (a 110000-page, 4.6 GB pool whose
    used pages sit at its end), through the block table and through sparse
    index lists; the oracle sees the same records in a compact pool."""
    import torch
    inp = W.make_inputs(3, 1, h_q, [700, 64, 1], pool=16, max_blocks=11, seed=29)
    rec = W.to_fp8_records(inp.kv_cache)
    n_pool, compact = 110000, rec.shape[0]
    high = n_pool - compact + np.arange(compact, dtype=np.int64)
    assert high[0] * 64 * W.FP8_RECORD > 2 ** 32
    dev = torch.device("cuda", 0)
    big = torch.zeros((n_pool, 64, 1, W.FP8_RECORD), dtype=torch.uint8, device=dev)
    big[torch.from_numpy(high).to(dev)] = torch.from_numpy(rec).to(dev)
    bt_high = high[inp.block_table].astype(np.int32)
    ref_out, ref_lse = ref_dense_fp8(inp, rec)
    tol = dense_out_bound(inp, kv=oracle.dequantize_fp8_cache(rec))
    print(f"[fp8 4 GiB] dense h_q={h_q}", flush=True)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, h_q, 1, fp8=True)
    out, lse = mla.mla_decode_fwd(_bf16(inp.q), big, _dev(bt_high), _dev(inp.cache_seqlens), inp.softmax_scale,
                                  sched, ns, fp8=True)
    torch.cuda.synchronize()
    assert_parity(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out,
                  ref_lse, f"fp8 pool past 4 GiB, dense h_q={h_q}", out_tol=tol)
    topk = 704
    idx = np.full((3, 1, topk), -1, dtype=np.int32)
    for i, L in enumerate(inp.cache_seqlens):
        t = np.arange(int(L))
        idx[i, 0, :L] = bt_high[i, t // 64] * 64 + t % 64
    print(f"[fp8 4 GiB] sparse h_q={h_q}", flush=True)
    ss, sn = mla.get_mla_metadata_sparse(None, 3, 1, h_q, topk)
    out2, lse2 = mla.mla_decode_sparse_fwd(_bf16(inp.q), big, _dev(idx), inp.softmax_scale, ss, sn, fp8=True)
    torch.cuda.synchronize()
    assert_parity(out2.float().cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64), ref_out,
                  ref_lse, f"fp8 pool past 4 GiB, sparse h_q={h_q}", out_tol=tol)
    del big
    torch.cuda.empty_cache()
