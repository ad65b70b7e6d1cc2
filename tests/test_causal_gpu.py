"""GPU parity for the causal mask of multi-token prediction (query token s of
s_q sees keys 0 .. L - s_q + s): the HIP path through the C ABI against the
oracle with causal=True, for every split-KV kernel (R <= 16, 16 < R < 128,
R >= 128 with one and with several 128-row groups), lengths around page
boundaries and below s_q (tokens that see no key), and forced splits (pieces
in which some rows see nothing)."""
import numpy as np
import pytest

from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, run_gpu

pytestmark = pytest.mark.gpu

LENS = [0, 1, 2, 3, 63, 64, 65, 66, 127, 128, 129, 200, 1000]


def _ref(inp):
    return oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                             causal=True)


@pytest.mark.parametrize("h_q,s_q", [(8, 2), (4, 3), (32, 2), (24, 3), (64, 2), (128, 2), (80, 2)])
@pytest.mark.parametrize("force", [0, 2])
def test_causal_edge_lengths(h_q, s_q, force):
    inp = W.make_inputs(len(LENS), s_q, h_q, LENS, pool=None, max_blocks=17, seed=100 + h_q * 10 + s_q)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp, force_splits=force, causal=True)
    assert_parity(out, lse, ref_out, ref_lse, f"causal h_q={h_q} s_q={s_q} force={force}",
                  out_tol=dense_out_bound(inp, causal=True))
    # Tokens that see no key: out = 0, lse = -inf.
    for b, L in enumerate(LENS):
        for s in range(s_q):
            if L - (s_q - 1 - s) <= 0:
                assert np.all(out[b, s] == 0) and np.all(np.isneginf(lse[b, :, s]))


def test_causal_single_query_token_matches_dense():
    inp = W.make_inputs(4, 1, 16, [70, 129, 1, 250], pool=None, max_blocks=4, seed=31)
    a = run_gpu(inp, force_splits=2)
    b = run_gpu(inp, force_splits=2, causal=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_mtp_shape_small_batch():
    # The ragged MTP workload's shape (s_q = 2, h_q = 128) on a smaller batch.
    inp = W.make_inputs(6, 2, 128, (512, 4096), pool=None, max_blocks=64, seed=44)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp, causal=True)
    assert_parity(out, lse, ref_out, ref_lse, "causal MTP shape", out_tol=dense_out_bound(inp, causal=True))
