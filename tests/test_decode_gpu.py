"""GPU parity tests: the HIP path through the C ABI against the CPU oracle on
the same seeded inputs, element by element, for the five workloads (full or
sampled), ragged and edge-case shapes, poisoned memory, the restart slow
path, page-permutation invariance and run-to-run determinism."""
import numpy as np
import pytest

from decode_attention_mla_amd import workloads as W
import oracle
from gpu_util import assert_parity, dense_out_bound, max_err, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _ref(inp, requests=None):
    return oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                             requests=requests)


@pytest.mark.parametrize("force", [0, 1, 2, 3])
def test_tiny_config(force):
    inp = W.config_inputs(1)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp, force_splits=force)
    assert_parity(out, lse, ref_out, ref_lse, f"config1 force_splits={force}")


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1)])
@pytest.mark.parametrize("force", [2, 3, 4, 5, 8, 9, 12, 17, 33])
def test_combine_over_every_chunk_size(h_q, s_q, force):
    """Every request cut into exactly `force` pieces: up to 8 pieces a pair a
    wave merges them (in chunks of 2, 4 or 8 by the count), above 8 the four
    waves of a workgroup take every fourth piece (1 to 9 pieces a wave, so
    every chunk size and a multi-chunk walk occur)."""
    lens = [64 * 40, 64 * 37 + 5, 64 * 35 - 3]
    inp = W.make_inputs(3, s_q, h_q, lens, pool=None, max_blocks=40, seed=900 + force)
    print(f"[combine] h_q={h_q} force={force}", flush=True)
    out, lse = run_gpu(inp, force_splits=force)
    ref_out, ref_lse = _ref(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"combine chunks h_q={h_q} force={force}", out_tol=dense_out_bound(inp))


def test_tiny_config_two_parts():
    # The other reading of "num_splits = 2": two parts, so only request 1 is cut.
    inp = W.config_inputs(1)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp, num_cus=2)
    assert_parity(out, lse, ref_out, ref_lse, "config1 two parts")


def test_memory_bound_config_full():
    inp = W.config_inputs(2)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp)
    assert_parity(out, lse, ref_out, ref_lse, "config2 full")


@pytest.mark.parametrize("idx", [3, 5])
def test_h128_configs_full(idx):
    inp = W.config_inputs(idx)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"config{idx} full")


@pytest.mark.parametrize("causal", [False, True])
def test_mtp_config_full(causal):
    """The ragged MTP workload (batch 128, s_q 2, h_q 128, L ~ U[512, 16384]),
    every output against the oracle, without and with the causal mask."""
    inp = W.config_inputs(4)
    print(f"[config4] causal={causal}: oracle", flush=True)
    ref_out, ref_lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                         causal=causal)
    print(f"[config4] causal={causal}: GPU", flush=True)
    out, lse = run_gpu(inp, causal=causal)
    assert_parity(out, lse, ref_out, ref_lse, f"config4 full causal={causal}")


@pytest.mark.parametrize("h_q", [16, 128])
def test_longest_request_sampled(h_q):
    """One request of 2^19 tokens (8192 pages, 604 MB of KV) beside a short
    one: the plan cuts it into about 256 pieces, whose partials the combine
    merges 64 to a wave; sampled heads match the oracle."""
    import decode_attention_mla_amd as mla
    L = 1 << 19
    inp = W.make_inputs(2, 1, h_q, [L, 100], pool=None, max_blocks=L // 64, seed=77)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, h_q, 1)
    pieces = int(ns[1].item() - ns[0].item())
    print(f"[longest] h_q={h_q} L={L} pieces={pieces}", flush=True)
    assert pieces >= 128
    out, lse = run_gpu(inp)
    picks = [(0, 0, h) for h in sorted({0, h_q // 2, h_q - 1})] + [(1, 0, 0)]
    ref_o, ref_l = oracle.mla_decode_rows(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens,
                                          inp.softmax_scale, picks)
    got_o = np.array([out[i, s, h] for i, s, h in picks])
    got_l = np.array([lse[i, h, s] for i, s, h in picks])
    assert_parity(got_o, got_l, ref_o, ref_l, f"longest request h_q={h_q}")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("h_q", [16, 128])
def test_large_batch_of_short_requests(h_q):
    """2048 requests of 0..300 tokens: parts span many requests (most pieces
    are whole requests, written straight to the output), some zero-length."""
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 301, size=2048).astype(np.int32)
    lens[::97] = 0
    inp = W.make_inputs(len(lens), 1, h_q, lens, pool=None, max_blocks=6, seed=91)
    print(f"[large batch] h_q={h_q} batch={len(lens)}", flush=True)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp)
    assert_parity(out, lse, ref_out, ref_lse, f"large batch h_q={h_q}", out_tol=dense_out_bound(inp))
    assert np.all(out[lens == 0] == 0) and np.all(np.isneginf(lse[lens == 0]))


@pytest.mark.parametrize("h_q", [16, 128])
def test_pages_beyond_4_gib_of_pool(h_q):
    """Pages at byte offsets past 2^32 of the KV pool (a 60000-page, 4.4 GB
    pool whose used pages sit at its end), through the block table and
    through sparse index lists: the 64-bit address arithmetic of both copy
    paths.  The oracle sees the same pages in a compact pool."""
    import torch
    import decode_attention_mla_amd as mla
    dev = torch.device("cuda", 0)
    inp = W.make_inputs(3, 1, h_q, [700, 64, 1], pool=16, max_blocks=11, seed=23)
    n_pool, compact = 60000, inp.kv_cache.shape[0]
    high = n_pool - compact + np.arange(compact, dtype=np.int64)      # compact page i -> pool page high[i]
    assert high[0] * 64 * 1152 > 2 ** 32
    big = torch.zeros((n_pool, 64, 1, W.D_QK), dtype=torch.bfloat16, device=dev)
    big[torch.from_numpy(high).to(dev)] = torch.from_numpy(inp.kv_cache.view(np.int16)).view(torch.bfloat16).to(dev)
    bt_high = high[inp.block_table].astype(np.int32)
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    sl = torch.from_numpy(inp.cache_seqlens).to(dev)
    ref_out, ref_lse = _ref(inp)
    tol = dense_out_bound(inp)
    print(f"[4 GiB] dense h_q={h_q}", flush=True)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, h_q, 1)
    out, lse = mla.mla_decode_fwd(q, big, torch.from_numpy(bt_high).to(dev), sl, inp.softmax_scale, sched, ns)
    torch.cuda.synchronize()
    assert_parity(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out,
                  ref_lse, f"pool past 4 GiB, dense h_q={h_q}", out_tol=tol)
    # the same keys as sparse lists: entry = pool page * 64 + slot
    topk = 704
    idx = np.full((3, 1, topk), -1, dtype=np.int32)
    for i, L in enumerate(inp.cache_seqlens):
        t = np.arange(int(L))
        idx[i, 0, :L] = bt_high[i, t // 64] * 64 + t % 64
    print(f"[4 GiB] sparse h_q={h_q}", flush=True)
    ss, sn = mla.get_mla_metadata_sparse(None, 3, 1, h_q, topk)
    out2, lse2 = mla.mla_decode_sparse_fwd(q, big, torch.from_numpy(idx).to(dev), inp.softmax_scale, ss, sn)
    torch.cuda.synchronize()
    assert_parity(out2.float().cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64), ref_out,
                  ref_lse, f"pool past 4 GiB, sparse h_q={h_q}", out_tol=tol)
    del big
    torch.cuda.empty_cache()


EDGE_LENS = [0, 1, 2, 63, 64, 65, 127, 128, 129, 200, 1000]


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (64, 2), (8, 1), (24, 1), (48, 2), (80, 2)])
@pytest.mark.parametrize("force", [0, 2])
def test_edge_lengths_and_head_counts(h_q, s_q, force):
    inp = W.make_inputs(len(EDGE_LENS), s_q, h_q, EDGE_LENS, pool=None, max_blocks=17, seed=h_q * 10 + s_q)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp, force_splits=force)
    assert_parity(out, lse, ref_out, ref_lse, f"edge lengths h_q={h_q} s_q={s_q} force={force}",
                  out_tol=dense_out_bound(inp))
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))     # L = 0


def test_many_parts_on_few_blocks():
    # More parts than blocks: most parts get nothing; requests of one block each.
    inp = W.make_inputs(5, 1, 128, [64, 1, 3, 64, 10], pool=None, max_blocks=1, seed=77)
    ref_out, ref_lse = _ref(inp)
    out, lse = run_gpu(inp)
    assert_parity(out, lse, ref_out, ref_lse, "tiny requests, 256 parts", out_tol=dense_out_bound(inp))


def test_nan_in_page_tails_and_unused_pages():
    inp = W.make_inputs(4, 1, 64, [70, 129, 1, 250], pool=20, max_blocks=4, seed=12, tail_poison=float("nan"))
    assert np.isnan(W.bf16_bits_to_f32(inp.kv_cache)).any()
    ref_out, ref_lse = _ref(inp)
    assert np.all(np.isfinite(ref_out))
    tol = dense_out_bound(inp)
    for force in (0, 2):
        out, lse = run_gpu(inp, force_splits=force)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        assert_parity(out, lse, ref_out, ref_lse, f"NaN tails force={force}", out_tol=tol)


@pytest.mark.parametrize("h_q", [16, 32, 128, 160])
def test_restart_when_later_page_outgrows_first_max(h_q):
    # First page scores ~0, a later page ~ +150 (far beyond the 2^64 headroom):
    # the kernel must take its restart path and still match.  At 128 and more
    # heads only rows 32 .. 63 outgrow their maxima (one wave of a 128-row
    # group votes for the restart of all four).
    rng = np.random.default_rng(3)
    L = 64 * 5 + 7
    keys = (0.01 * rng.standard_normal((L, W.D_QK))).astype(np.float32)
    keys[64 * 3 + 5, :] = 0.5          # one token with a huge score
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
    ref_out, ref_lse = _ref(inp)
    assert ref_lse.max() > 100
    tol = dense_out_bound(inp)
    for force in (0, 1):
        out, lse = run_gpu(inp, force_splits=force)
        assert_parity(out, lse, ref_out, ref_lse, f"restart path force={force}", out_tol=tol)


def test_identical_scores_closed_form_on_gpu():
    rng = np.random.default_rng(21)
    L = 300
    inp = W.make_inputs(1, 1, 16, [L], pool=8, max_blocks=5, seed=21)
    kv = inp.kv_cache.copy()
    rope = rng.standard_normal(64).astype(np.float32)
    for t in range(L):
        row = rng.standard_normal(W.D_QK).astype(np.float32)
        row[512:] = rope
        kv[inp.block_table[0, t // 64], t % 64, 0] = W.f32_to_bf16_bits(row)
    q = rng.standard_normal((1, 1, 16, W.D_QK)).astype(np.float32)
    q[..., :512] = 0
    inp.kv_cache, inp.q = kv, W.f32_to_bf16_bits(q)
    out, lse = run_gpu(inp)
    vals = np.stack([W.bf16_bits_to_f32(kv[inp.block_table[0, t // 64], t % 64, 0, :512]) for t in range(L)])
    mean_v = vals.astype(np.float64).mean(axis=0)
    qr = W.bf16_bits_to_f32(inp.q[0, 0, :, 512:]).astype(np.float64)
    expect_lse = inp.softmax_scale * (qr @ W.bf16_bits_to_f32(W.f32_to_bf16_bits(rope)).astype(np.float64)) + np.log(L)
    assert max_err(out[0, 0], np.broadcast_to(mean_v, (16, 512))) <= 1e-2
    assert max_err(lse[0, :, 0], expect_lse) <= 1e-3


def test_page_permutation_is_bitwise_invariant_and_deterministic():
    inp = W.config_inputs(2)
    out1, lse1 = run_gpu(inp)
    out1b, lse1b = run_gpu(inp)
    assert np.array_equal(out1, out1b) and np.array_equal(lse1, lse1b), "run-to-run difference"
    perm = np.random.default_rng(9).permutation(inp.num_blocks)
    kv2 = np.empty_like(inp.kv_cache)
    kv2[perm] = inp.kv_cache
    inp2 = W.MlaInputs(inp.name, inp.q, kv2, perm[inp.block_table].astype(np.int32), inp.cache_seqlens,
                       inp.softmax_scale)
    out2, lse2 = run_gpu(inp2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2), "page permutation changed the result"


def test_plan_reuse_across_calls_and_scale_zero():
    import torch
    import decode_attention_mla_amd as mla
    inp = W.config_inputs(1)
    d = to_device(inp)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q)
    ref_out, ref_lse = oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, 0.0)
    for _ in range(3):    # one plan, several "layers"
        out, lse = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], 0.0, sched, ns)
    torch.cuda.synchronize()
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, "scale 0, reused plan")


def test_python_argument_checks():
    import torch
    import decode_attention_mla_amd as mla
    inp = W.config_inputs(1)
    d = to_device(inp)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q)
    with pytest.raises(ValueError, match="bfloat16"):
        mla.mla_decode_fwd(d["q"].float(), d["kv"], d["bt"], d["sl"], 0.1, sched, ns)
    with pytest.raises(ValueError, match="num_splits"):
        mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], 0.1, sched, ns[:-1])
    with pytest.raises(ValueError, match="workspace"):
        mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], 0.1, sched, ns,
                           workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("case", ["config2", "h64_sq2_forced_splits"])
def test_graph_replay_matches_eager(case):
    """One decode call captured in a HIP graph and replayed several times,
    with eager work (clearing the outputs) and synchronisation between the
    replays: every replay must reproduce the eager result bit for bit."""
    import torch
    import decode_attention_mla_amd as mla
    if case == "config2":
        inp, force = W.config_inputs(2), 0
    else:
        inp, force = W.make_inputs(6, 2, 64, [70, 129, 1000, 0, 640, 300], pool=None, max_blocks=16, seed=31), 3
    d = to_device(inp)
    sched, ns = mla.get_mla_metadata(inp.cache_seqlens, inp.h_q, inp.s_q, force_splits=force)
    ref_out, ref_lse = mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns)
    torch.cuda.synchronize()
    ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
    out, lse = torch.empty_like(ref_out), torch.empty_like(ref_lse)
    ws = torch.empty(mla.mla_workspace_bytes(sched.shape[0] + inp.batch - 1, inp.h_q, inp.s_q),
                     dtype=torch.uint8, device=out.device)

    def call():
        mla.mla_decode_fwd(d["q"], d["kv"], d["bt"], d["sl"], inp.softmax_scale, sched, ns, out=out, lse=lse,
                           workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    for _ in range(4):
        out.zero_()
        lse.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
