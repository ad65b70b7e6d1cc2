"""GPU tests of plans that carry each part's first page (column 6, from
mla_plan_attach_pages or the device planner given the block table): decode
results equal those of the plain plan bit for bit on every kernel (only the
16-row kernel reads the column), for bf16 and FP8 caches, ragged and empty
requests and forced splits; the device planner's column equals the host
attachment; and a captured planner + decode step follows new lengths and a
rewritten block table between replays."""
import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, to_device

pytestmark = pytest.mark.gpu


CASES = [
    # h_q, s_q, lengths, force_splits, causal, fp8
    (16, 1, [100, 257, 0, 640, 1, 64], 0, False, False),
    (16, 1, [100, 257, 0, 640, 1, 64], 0, False, True),
    (16, 1, [1000, 0, 2000, 65], 3, False, False),
    (16, 1, [1000, 0, 2000, 65], 3, False, True),
    (8, 2, [70, 300, 0, 129], 2, True, False),
    (8, 2, [70, 300, 0, 129], 0, True, True),
    (128, 1, [64, 0, 300, 1100], 2, False, False),
    (128, 2, [129, 700], 0, True, True),
]


def _decode(inp, d, kv, sched, ns, causal, fp8):
    import torch
    out, lse = mla.mla_decode_fwd(d["q"], kv, d["bt"], d["sl"], inp.softmax_scale, sched, ns, causal=causal,
                                  fp8=fp8)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attached_plan_is_bitwise_the_plain_plan(case):
    import torch
    h_q, s_q, lens, force, causal, fp8 = CASES[case]
    print(f"[attach] case {case}: h_q={h_q} s_q={s_q} lens={lens} force={force} causal={causal} fp8={fp8}",
          flush=True)
    max_blocks = -(-max(lens) // 64) + 1
    inp = W.make_inputs(len(lens), s_q, h_q, lens, pool=len(lens) * max_blocks + 5, max_blocks=max_blocks,
                        seed=700 + case)
    pool = inp.kv_cache.shape[0]
    d = to_device(inp)
    rec = W.to_fp8_records(inp.kv_cache) if fp8 else None
    kv = torch.from_numpy(rec).cuda() if fp8 else d["kv"]
    plain_s, plain_n = mla.get_mla_metadata(inp.cache_seqlens, h_q, s_q, force_splits=force, fp8=fp8)
    att_s, att_n = mla.get_mla_metadata(inp.cache_seqlens, h_q, s_q, force_splits=force, fp8=fp8,
                                        block_table=inp.block_table, num_blocks=pool)
    hs = att_s.cpu().numpy()
    assert np.array_equal(hs[:, [0, 1, 2, 3, 4, 5, 7]], plain_s.cpu().numpy()[:, [0, 1, 2, 3, 4, 5, 7]])
    assert np.any(hs[:, 6] > 0)
    a_out, a_lse = _decode(inp, d, kv, plain_s, plain_n, causal, fp8)
    b_out, b_lse = _decode(inp, d, kv, att_s, att_n, causal, fp8)
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    assert torch.equal(a_lse.view(torch.int32), b_lse.view(torch.int32))
    kv_ref = oracle.dequantize_fp8_cache(rec) if fp8 else inp.kv_cache
    ref_out, ref_lse = oracle.mla_decode(inp.q, kv_ref, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                         causal=causal)
    assert_parity(b_out.float().cpu().numpy().astype(np.float64), b_lse.cpu().numpy().astype(np.float64),
                  ref_out, ref_lse, f"attached plan case {case}", out_tol=dense_out_bound(inp, causal, kv_ref))


@pytest.mark.parametrize("h_q,s_q,seed", [(16, 1, 0), (16, 1, 1), (128, 2, 2), (8, 1, 3)])
def test_device_plan_with_table_equals_host_attachment(h_q, s_q, seed):
    import torch
    rng = np.random.default_rng(800 + seed)
    b = int(rng.choice([5, 64, 300]))
    sl = rng.integers(0, 6000, size=b).astype(np.int32)
    sl[rng.random(b) < 0.2] = 0
    max_blocks = int(-(-sl.max() // 64)) + 2
    num_blocks = b * max_blocks
    table = rng.permutation(num_blocks).astype(np.int32).reshape(b, max_blocks)
    table[0, 0] = num_blocks + 3          # an id outside the pool: the device planner leaves it unattached
    ds, dn = mla.get_mla_metadata_device(torch.from_numpy(sl).cuda(), h_q, s_q,
                                         block_table=torch.from_numpy(table).cuda(), num_blocks=num_blocks)
    torch.cuda.synchronize()
    ds, dn = ds.cpu().numpy(), dn.cpu().numpy()
    hs, hn, _ = mla.get_mla_metadata_host(sl, h_q, s_q)
    n = hs.shape[0]
    ok = table.copy()
    ok[0, 0] = 0
    mla.binding.attach_pages(hs, sl, ok, num_blocks)
    if sl[0] > 0:
        assert hs[0, 6] == 1
        hs[0, 6] = 0                      # the device planner's reading of the out-of-pool id
    assert np.array_equal(dn, hn)
    assert np.array_equal(ds[:n], hs)
    assert np.all(ds[n:, 6] == 0)


def test_graph_with_attached_device_plan_follows_lengths_and_table():
    """Capture planner (given the table) + decode once; before each replay
    write new lengths and a new block table into the captured buffers."""
    import torch
    steps = [[70, 129, 1, 250, 64], [71, 130, 0, 251, 65], [200, 3, 640, 252, 128], [0, 1000, 641, 5, 129]]
    h_q, s_q = 16, 1
    max_blocks = 17
    # every page holds ordinary finite values (no poisoned tails), so that
    # any table the replays write names valid keys
    inp = W.make_inputs(5, s_q, h_q, [max(x) for x in zip(*steps)], pool=5 * max_blocks, max_blocks=max_blocks,
                        seed=91, tail_poison=0.375)
    pool = inp.kv_cache.shape[0]
    d = to_device(inp)
    b = inp.batch
    out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device="cuda")
    sched0, _ = mla.get_mla_metadata_device(d["sl"], h_q, s_q)
    ws = torch.empty(mla.mla_workspace_bytes(sched0.shape[0] + b - 1, h_q, s_q), dtype=torch.uint8, device="cuda")

    def step():
        sched, ns = mla.get_mla_metadata_device(d["sl"], h_q, s_q, block_table=d["bt"], num_blocks=pool)
        mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns, out=out, lse=lse,
                           workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for lens in steps:
        table = rng.permutation(pool)[:b * max_blocks].astype(np.int32).reshape(b, max_blocks)
        d["sl"].copy_(torch.tensor(lens, dtype=torch.int32, device="cuda"))
        d["bt"].copy_(torch.from_numpy(table).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        inp.cache_seqlens = np.array(lens, dtype=np.int32)
        inp.block_table = table
        ref_out, ref_lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                             inp.softmax_scale)
        got_out = out.float().cpu().numpy().astype(np.float64)
        got_lse = lse.cpu().numpy().astype(np.float64)
        assert_parity(got_out, got_lse, ref_out, ref_lse, f"graph replay lens={lens}", out_tol=dense_out_bound(inp))
