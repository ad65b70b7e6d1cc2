"""The allocation-free entry point (mla_decode_fwd_noalloc) through the C ABI
against mla_decode_fwd: same plan, same kernels, so the outputs must agree
bit for bit; two calls in a row on the library's one per-GPU array, the
second on a smaller input (which must not see the first call's partials),
and a plan too large for the array rejected before any launch."""
import ctypes

import numpy as np
import pytest

import decode_attention_mla_amd as mla
from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, to_device

pytestmark = pytest.mark.gpu


def _both(inp, force=0, causal=False):
    import torch
    d = to_device(inp)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, force_splits=force)
    print(f"[no-alloc] b={inp.batch} s_q={inp.s_q} h_q={inp.h_q} parts={sched.shape[0]} force={force} "
          f"causal={causal}", flush=True)
    ref_out, ref_lse = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns,
                                          causal=causal)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    mla.mla_decode_fwd_noalloc(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns, out, lse,
                               causal=causal)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    import torch
    # Call 1: the memory-bound workload (219 pieces, every request split).
    big = W.config_inputs(2)
    out, lse, ref_out, ref_lse = _both(big)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    o_ref, l_ref = oracle.mla_decode(big.q, big.kv_cache, big.block_table, big.cache_seqlens, big.softmax_scale)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "no-alloc, memory-bound workload")
    # Call 2, right after on the same array: a smaller input, forced splits, causal, h_q 128.
    small = W.make_inputs(5, 2, 64, [70, 129, 1000, 0, 300], pool=None, max_blocks=17, seed=12)
    out, lse, ref_out, ref_lse = _both(small, force=3, causal=True)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    o_ref, l_ref = oracle.mla_decode(small.q, small.kv_cache, small.block_table, small.cache_seqlens,
                                     small.softmax_scale, causal=True)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "no-alloc, second smaller call",
                  out_tol=dense_out_bound(small, causal=True))


def test_noalloc_rejects_plans_larger_than_the_array():
    L = mla.lib()
    dummy = ctypes.c_void_p(16)   # never dereferenced: the size check fails before any HIP call
    # 4096 parts x 128 heads x 2 query tokens: far more partial slots than the array holds
    rc = L.mla_decode_fwd_noalloc(dummy, dummy, dummy, dummy, 64, 2, 128, 8, 4, 0.1, 0, 0, dummy, 4096, dummy,
                                  dummy, dummy, None)
    assert rc == -3 and b"split workspace" in L.mla_last_error()
    need = mla.mla_workspace_bytes(4096 + 64 - 1, 128, 2)
    assert need > (128 << 20)
