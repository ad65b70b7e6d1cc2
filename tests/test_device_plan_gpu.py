"""GPU tests of the device-side planner (mla_get_metadata_device): its table
equals the host planner's walk bit for bit (plus empty rows up to the part
count), decode results with it equal those with the host plan, and a HIP
graph holding planner + decode replans correctly when the lengths in device
memory change between replays."""
import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _device_plan(seqlens, h_q, s_q, num_cus=0):
    import torch
    sl = torch.from_numpy(np.asarray(seqlens, dtype=np.int32)).cuda()
    sched, ns = mla.get_mla_metadata_device(sl, h_q, s_q, num_cus=num_cus)
    torch.cuda.synchronize()
    return sched.cpu().numpy(), ns.cpu().numpy()


@pytest.mark.parametrize("seed", range(24))
def test_device_plan_equals_host_walk(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.choice([1, 3, 16, 64, 65, 100, 130, 300, 1000]))
    h_q, s_q = [(16, 1), (128, 1), (128, 2), (32, 2), (8, 1)][seed % 5]
    kind = seed % 4
    if kind == 0:
        sl = rng.integers(0, 5000, size=b)
    elif kind == 1:
        sl = rng.integers(0, 130, size=b)                  # tiny requests: the walk ends before the last part
    elif kind == 2:
        sl = np.where(rng.random(b) < 0.3, 0, rng.integers(1, 70000, size=b))
    else:
        sl = np.full(b, int(rng.integers(1, 20000)))
    sl = sl.astype(np.int32)
    num_cus = int(rng.choice([0, 1, 2, 3, 37, 256, 1024]))
    ds, dn = _device_plan(sl, h_q, s_q, num_cus=num_cus)
    hs, hn, total = mla.get_mla_metadata_host(sl, h_q, s_q, num_cus=num_cus)
    np_host = hs.shape[0]
    assert np.array_equal(dn, hn), (dn, hn)
    assert np.array_equal(ds[:np_host], hs)
    assert np.all(ds[np_host:, 0] == 1) and np.all(ds[np_host:, 1] == 0)   # empty rows
    assert np.all(ds[:, 5] == hs[0, 5])
    assert total == dn[-1] <= ds.shape[0] + b - 1


@pytest.mark.parametrize("num_cus", [1, 3, 256])
def test_device_plan_equals_host_walk_beyond_32_bits(num_cus):
    """Lengths near 2^31 in a large batch: block totals and the payload pass
    2^32, so the walk's capacity arithmetic must be 64-bit."""
    rng = np.random.default_rng(num_cus)
    sl = (2**31 - 1 - rng.integers(0, 2**20, size=5000)).astype(np.int32)
    sl[::7] = rng.integers(0, 100, size=sl[::7].shape[0])
    ds, dn = _device_plan(sl, 16, 1, num_cus=num_cus)
    hs, hn, _ = mla.get_mla_metadata_host(sl, 16, 1, num_cus=num_cus)
    assert np.array_equal(dn, hn)
    assert np.array_equal(ds[:hs.shape[0]], hs)


def test_decode_with_device_plan_equals_host_plan():
    import torch
    inp = W.config_inputs(2)
    d = to_device(inp)
    hs, hn = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q)
    ds, dn = mla.get_mla_metadata_device(d["sl"], inp.h_q, inp.s_q)
    a = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, hs, hn)
    b = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, ds, dn)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 2)])
def test_graph_replans_when_device_lengths_change(h_q, s_q):
    """Capture planner + decode once; before each replay write new lengths
    into the captured length buffer (as a serving loop appends tokens)."""
    import torch
    steps = [[70, 129, 1, 250, 64], [71, 130, 2, 251, 65], [200, 3, 640, 252, 128], [0, 1000, 641, 5, 129]]
    inp = W.make_inputs(5, s_q, h_q, [max(x) for x in zip(*steps)], pool=None, max_blocks=17, seed=61)
    d = to_device(inp)
    sl_dev = d["sl"]
    b = inp.batch
    out = torch.empty((b, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device="cuda")
    # Buffers sized for any lengths: parts from the policy, workspace for parts + b - 1 slots.
    sched0, ns0 = mla.get_mla_metadata_device(sl_dev, h_q, s_q)
    ws = torch.empty(mla.mla_workspace_bytes(sched0.shape[0] + b - 1, h_q, s_q), dtype=torch.uint8, device="cuda")

    def step():
        sched, ns = mla.get_mla_metadata_device(sl_dev, h_q, s_q)
        mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], sl_dev, inp.softmax_scale, sched, ns, out=out, lse=lse,
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
    for lens in steps:
        sl_dev.copy_(torch.tensor(lens, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        inp.cache_seqlens = np.array(lens, dtype=np.int32)
        ref_out, ref_lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                             inp.softmax_scale)
        got_out = out.float().cpu().numpy().astype(np.float64)
        got_lse = lse.cpu().numpy().astype(np.float64)
        assert_parity(got_out, got_lse, ref_out, ref_lse, f"graph replay lens={lens}", out_tol=dense_out_bound(inp))
